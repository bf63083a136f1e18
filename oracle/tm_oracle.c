/*
 * tm_oracle.c -- fp64 CPU oracle for the 2-D TM Maxwell FDTD propagator,
 * its exact discrete adjoint and the model gradients dJ/dCa, dJ/dCb.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links
 * or loads this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code with the GPU path.
 *
 * What it follows (source page: tide-GPR 0.0.9, tide/csrc/maxwell.cu):
 *   - the header comment's discrete forward equations
 *       Ey <- Ca Ey + Cb (Dx[Hz] - Dz[Hx]),
 *       Hx <- Hx - Cq Dz^h[Ey],   Hz <- Hz + Cq Dx^h[Ey];
 *   - the per-step order of the host launcher ``forward``: H half-step,
 *     E step, source injection (raw add), receiver recording;
 *   - the index ranges and CPML band flags of ``forward_kernel_h`` and
 *     ``forward_kernel_e`` (E cells P..n-P on each axis, Hx rows up to
 *     ny-P-1, Hz columns up to nx-P-1, H flags outside [lo, hi-1), E flags
 *     outside [lo, hi));
 *   - the CPML recursion m <- b m + a d, d <- d / kappa + m;
 *   - the snapshot timing of ``forward_kernel_e_with_storage`` (Ey before
 *     the update, curl H after its CPML correction);
 *   - the gradient definitions of the header comment
 *     (dJ/dCa = sum_n Ey^n lambda^{n+1}, dJ/dCb = sum_n curlH^n lambda^{n+1}),
 *     masked to the interior window as in the kernels' gradient branch;
 *   - the reverse loop order of ``backward``: residual injected at the
 *     receivers first, then the adjoint field read at the sources.
 *
 * Readings where the page is silent (its stencil header is not on the page):
 *   - staggered Taylor coefficients c_k; the half-point derivative at
 *     x+1/2 (stored at x) is rdx sum_k c_k (F[x+k] - F[x-k+1]) and the
 *     integer-point derivative is rdx sum_k c_k (F[x+k-1] - F[x-k]);
 *   - a field is zero outside its update set and never written there;
 *   - the adjoint is the exact transpose of the forward step, CPML
 *     included: coefficient at the source point, then that point's CPML
 *     filter run backwards in time on its own memory, then the transposed
 *     stencil.  (The page's kernels apply Cb, Cq and the destination CPML
 *     outside the stencil, which is the transpose only for uniform
 *     coefficients away from the bands.)
 *   - duplicate source (receiver) cells of one shot add up; a negative
 *     index is skipped and records (adjoint source reads) 0.
 *
 * Storage: every field is a full [S][ny][nx] fp64 array, CPML memories
 * included.  Snapshots cover the interior window only.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef long long ll;

typedef struct {
    int order;          /* 2, 4 or 8 */
    int periodic;       /* test-only: wrap-around indices, all cells updated, no CPML */
    ll n_shots, ny, nx;
    ll pml_y0, pml_y1, pml_x0, pml_x1;
    double rdy, rdx;    /* 1/dy, 1/dx */
    ll n_src, n_rec;
} orc_geom;

/* Staggered-grid Taylor coefficients c_1..c_P. */
static int coefs(int order, double *c)
{
    switch (order) {
    case 2: c[0] = 1.0; return 1;
    case 4: c[0] = 9.0 / 8.0; c[1] = -1.0 / 24.0; return 2;
    case 8:
        c[0] = 1225.0 / 1024.0; c[1] = -245.0 / 3072.0;
        c[2] = 49.0 / 5120.0;   c[3] = -5.0 / 7168.0;
        return 4;
    default: return -1;
    }
}

int orc_coefficients(int order, double *c) { return coefs(order, c); }

/* Threads an OpenMP parallel region of the oracle uses (1 without OpenMP). */
#ifdef _OPENMP
#include <omp.h>
int orc_num_threads(void) { return omp_get_max_threads(); }
#else
int orc_num_threads(void) { return 1; }
#endif

/* ---- geometry helpers ---------------------------------------------------- */

typedef struct {
    const orc_geom *g;
    int P;
    double c[4];
} ctx_t;

static ll wrap(ll i, ll n) { i %= n; return i < 0 ? i + n : i; }

/* cell (y, x) of one shot's slab, with wrap-around in periodic mode */
static double at(const ctx_t *k, const double *F, ll y, ll x)
{
    const orc_geom *g = k->g;
    if (g->periodic) { y = wrap(y, g->ny); x = wrap(x, g->nx); }
    return F[y * g->nx + x];
}

static int in_e(const ctx_t *k, ll y, ll x)
{
    const orc_geom *g = k->g;
    if (g->periodic) return 1;
    return y >= k->P && y <= g->ny - k->P && x >= k->P && x <= g->nx - k->P;
}
static int in_hx(const ctx_t *k, ll y, ll x)
{
    const orc_geom *g = k->g;
    if (g->periodic) return 1;
    return y >= k->P && y <= g->ny - k->P - 1 && x >= k->P && x <= g->nx - k->P;
}
static int in_hz(const ctx_t *k, ll y, ll x)
{
    const orc_geom *g = k->g;
    if (g->periodic) return 1;
    return y >= k->P && y <= g->ny - k->P && x >= k->P && x <= g->nx - k->P - 1;
}

/* CPML band flags: E points outside [lo, hi); H points outside [lo, max(lo, hi-1)). */
static int flag_e(const ctx_t *k, ll i, ll lo, ll hi) { return !k->g->periodic && (i < lo || i >= hi); }
static int flag_h(const ctx_t *k, ll i, ll lo, ll hi)
{
    ll hh = hi - 1 > lo ? hi - 1 : lo;
    return !k->g->periodic && (i < lo || i >= hh);
}
static int interior(const orc_geom *g, ll y, ll x)
{
    return y >= g->pml_y0 && y < g->pml_y1 && x >= g->pml_x0 && x < g->pml_x1;
}

/* ---- stencils ------------------------------------------------------------ */
/* half-point y derivative (Hx point y+1/2, stored at y) of an integer-point field */
static double d_yh(const ctx_t *k, const double *F, ll y, ll x)
{
    double s = 0.0;
    for (int q = 1; q <= k->P; ++q) s += k->c[q - 1] * (at(k, F, y + q, x) - at(k, F, y - q + 1, x));
    return k->g->rdy * s;
}
static double d_xh(const ctx_t *k, const double *F, ll y, ll x)
{
    double s = 0.0;
    for (int q = 1; q <= k->P; ++q) s += k->c[q - 1] * (at(k, F, y, x + q) - at(k, F, y, x - q + 1));
    return k->g->rdx * s;
}
/* integer-point y derivative of a half-point field */
static double d_y(const ctx_t *k, const double *F, ll y, ll x)
{
    double s = 0.0;
    for (int q = 1; q <= k->P; ++q) s += k->c[q - 1] * (at(k, F, y + q - 1, x) - at(k, F, y - q, x));
    return k->g->rdy * s;
}
static double d_x(const ctx_t *k, const double *F, ll y, ll x)
{
    double s = 0.0;
    for (int q = 1; q <= k->P; ++q) s += k->c[q - 1] * (at(k, F, y, x + q - 1) - at(k, F, y, x - q));
    return k->g->rdx * s;
}

/* CPML filter: memory m <- b m + a d; output d / kappa + m. */
static double cpml(double *m, double a, double b, double kappa, double d)
{
    *m = b * (*m) + a * d;
    return d / kappa + *m;
}

/* CPML array rows in the packed [12][L] layout */
enum { AY, BY, KY, AYH, BYH, KYH, AX, BX, KX, AXH, BXH, KXH };

static int setup(ctx_t *k, const orc_geom *g)
{
    memset(k, 0, sizeof(*k));
    k->g = g;
    k->P = coefs(g->order, k->c);
    if (k->P < 0) return -1;
    if (g->ny < 2 * k->P + 2 || g->nx < 2 * k->P + 2) return -2;
    return 0;
}

/* ---- forward ------------------------------------------------------------- */
/*
 * Runs steps t0..t1-1 on the state (E, Hx, Hz and the four CPML memories
 * psi_ez [Hx update], psi_ex [Hz update], psi_hxz and psi_hzx [E update],
 * each [S][ny][nx]), which the caller owns and may carry between calls.
 *   f    [nt][S][n_src]   source amplitudes (indexed by absolute step)
 *   r    [nt][S][n_rec]   records (written for the steps run), may be NULL
 *   snap_e, snap_c  [..][S][ny_i][nx_i] Ey^n and curlH^n on the interior
 *                   window, step n at index n - snap_t0 (written for the
 *                   steps run), may be NULL
 */
int orc_forward(const orc_geom *g, const double *ca, const double *cb, const double *cq,
                const double *cpml_arr, ll cpml_len,
                const double *f, const ll *src, const ll *rec,
                double *E, double *Hx, double *Hz,
                double *psi_ez, double *psi_ex, double *psi_hxz, double *psi_hzx,
                double *r, double *snap_e, double *snap_c, ll snap_t0, ll t0, ll t1)
{
    ctx_t k;
    int rc = setup(&k, g);
    if (rc) return rc;
    const ll ny = g->ny, nx = g->nx, S = g->n_shots, numel = ny * nx;
    const ll nyi = g->pml_y1 - g->pml_y0, nxi = g->pml_x1 - g->pml_x0;
    const double *cp = cpml_arr;
#define CP(row, i) cp[(ll)(row) * cpml_len + (i)]

    for (ll n = t0; n < t1; ++n) {
        for (ll s = 0; s < S; ++s) {
            double *e = E + s * numel, *hx = Hx + s * numel, *hz = Hz + s * numel;
            double *pez = psi_ez + s * numel, *pex = psi_ex + s * numel;
            double *phxz = psi_hxz + s * numel, *phzx = psi_hzx + s * numel;

            /* H half-step: Hx -= Cq * Dz^h Ey ; Hz += Cq * Dx^h Ey */
#pragma omp parallel for schedule(static)
            for (ll y = 0; y < ny; ++y) {
                for (ll x = 0; x < nx; ++x) {
                    ll j = y * nx + x;
                    if (in_hx(&k, y, x)) {
                        double d = d_yh(&k, e, y, x);
                        if (flag_h(&k, y, g->pml_y0, g->pml_y1))
                            d = cpml(&pez[j], CP(AYH, y), CP(BYH, y), CP(KYH, y), d);
                        hx[j] = hx[j] - cq[j] * d;
                    }
                    if (in_hz(&k, y, x)) {
                        double d = d_xh(&k, e, y, x);
                        if (flag_h(&k, x, g->pml_x0, g->pml_x1))
                            d = cpml(&pex[j], CP(AXH, x), CP(BXH, x), CP(KXH, x), d);
                        hz[j] = hz[j] + cq[j] * d;
                    }
                }
            }

            /* E step: Ey = Ca Ey + Cb (Dx Hz - Dz Hx) */
#pragma omp parallel for schedule(static)
            for (ll y = 0; y < ny; ++y) {
                for (ll x = 0; x < nx; ++x) {
                    if (!in_e(&k, y, x)) continue;
                    ll j = y * nx + x;
                    double u = d_x(&k, hz, y, x);
                    if (flag_e(&k, x, g->pml_x0, g->pml_x1))
                        u = cpml(&phzx[j], CP(AX, x), CP(BX, x), CP(KX, x), u);
                    double v = d_y(&k, hx, y, x);
                    if (flag_e(&k, y, g->pml_y0, g->pml_y1))
                        v = cpml(&phxz[j], CP(AY, y), CP(BY, y), CP(KY, y), v);
                    double curl = u - v;
                    if (!g->periodic && interior(g, y, x)) {
                        ll w = (((n - snap_t0) * S + s) * nyi + (y - g->pml_y0)) * nxi + (x - g->pml_x0);
                        if (snap_e) snap_e[w] = e[j];
                        if (snap_c) snap_c[w] = curl;
                    }
                    e[j] = ca[j] * e[j] + cb[j] * curl;
                }
            }

            /* sources, then receivers */
            for (ll i = 0; i < g->n_src; ++i) {
                ll c = src[s * g->n_src + i];
                if (c >= 0) e[c] += f[(n * S + s) * g->n_src + i];
            }
            if (r) {
                for (ll i = 0; i < g->n_rec; ++i) {
                    ll c = rec[s * g->n_rec + i];
                    r[(n * S + s) * g->n_rec + i] = c >= 0 ? e[c] : 0.0;
                }
            }
        }
    }
#undef CP
    return 0;
}

/* ---- exact adjoint -------------------------------------------------------- */
/*
 * Reverse steps n = t1-1 .. t0 of the exact transpose of orc_forward's step,
 * on an adjoint state the caller owns and may carry between calls (all
 * [S][ny][nx]: lambda_E, lambda_Hx, lambda_Hz and the adjoint memories of
 * the four CPML filters; zero before the last step nt-1).
 *   grad_r  [nt][S][n_rec]  dJ/dr (indexed by absolute step)
 *   grad_f  [nt][S][n_src]  dJ/df (rows t0..t1-1 written, may be NULL)
 *   snap_e, snap_c  interior snapshots from orc_forward, step n at index
 *                   n - snap_t0 (may be NULL: no gradient is accumulated)
 *   gca, gcb  [S][ny][nx]  per-shot gradients, accumulated (+=) on the
 *                          interior window; may be NULL
 */
int orc_adjoint_range(const orc_geom *g, const double *ca, const double *cb, const double *cq,
                      const double *cpml_arr, ll cpml_len,
                      const ll *src, const ll *rec,
                      const double *grad_r, double *grad_f,
                      const double *snap_e, const double *snap_c, ll snap_t0,
                      double *lE_all, double *lHx_all, double *lHz_all,
                      double *m_hzx_all, double *m_hxz_all, double *m_ex_all, double *m_ez_all,
                      double *gca, double *gcb, ll t0, ll t1)
{
    ctx_t k;
    int rc = setup(&k, g);
    if (rc) return rc;
    if (g->periodic) return -3;
    const ll ny = g->ny, nx = g->nx, S = g->n_shots, numel = ny * nx;
    const ll nyi = g->pml_y1 - g->pml_y0, nxi = g->pml_x1 - g->pml_x0;
    const double *cp = cpml_arr;
#define CP(row, i) cp[(ll)(row) * cpml_len + (i)]

    double *U = calloc((size_t)numel, sizeof(double));     /* filtered Cb*lambda for the Hz transpose */
    double *W = calloc((size_t)numel, sizeof(double));     /* ... for the Hx transpose */
    double *TZ = calloc((size_t)numel, sizeof(double));    /* filtered Cq*lambda_Hz */
    double *TX = calloc((size_t)numel, sizeof(double));    /* filtered Cq*lambda_Hx */
    if (!U || !W || !TZ || !TX) {
        rc = -4;
        goto done;
    }

    for (ll s = 0; s < S; ++s) {
        double *lE = lE_all + s * numel, *lHx = lHx_all + s * numel, *lHz = lHz_all + s * numel;
        double *m_hzx = m_hzx_all + s * numel; /* adjoint memory of the E-update x filter */
        double *m_hxz = m_hxz_all + s * numel; /* ... E-update y filter */
        double *m_ex = m_ex_all + s * numel;   /* ... Hz-update x filter */
        double *m_ez = m_ez_all + s * numel;   /* ... Hx-update y filter */
        double *ga = gca ? gca + s * numel : NULL;
        double *gb = gcb ? gcb + s * numel : NULL;

        for (ll n = t1 - 1; n >= t0; --n) {
            /* transpose of the receiver read: inject the residual */
            for (ll i = 0; i < g->n_rec; ++i) {
                ll c = rec[s * g->n_rec + i];
                if (c >= 0) lE[c] += grad_r[(n * S + s) * g->n_rec + i];
            }
            /* transpose of the source add: read the adjoint field */
            if (grad_f) {
                for (ll i = 0; i < g->n_src; ++i) {
                    ll c = src[s * g->n_src + i];
                    grad_f[(n * S + s) * g->n_src + i] = c >= 0 ? lE[c] : 0.0;
                }
            }

            /* transpose of the E step: gradient, coefficient, filters */
#pragma omp parallel for schedule(static)
            for (ll y = 0; y < ny; ++y) {
                for (ll x = 0; x < nx; ++x) {
                    ll j = y * nx + x;
                    if (!in_e(&k, y, x)) { U[j] = 0.0; W[j] = 0.0; continue; }
                    double e = lE[j];
                    if (interior(g, y, x)) {
                        ll w = (((n - snap_t0) * S + s) * nyi + (y - g->pml_y0)) * nxi + (x - g->pml_x0);
                        if (ga && snap_e) ga[j] += e * snap_e[w];
                        if (gb && snap_c) gb[j] += e * snap_c[w];
                    }
                    double h = cb[j] * e;
                    double u = h, w = h;
                    if (flag_e(&k, x, g->pml_x0, g->pml_x1))
                        u = cpml(&m_hzx[j], CP(AX, x), CP(BX, x), CP(KX, x), h);
                    if (flag_e(&k, y, g->pml_y0, g->pml_y1))
                        w = cpml(&m_hxz[j], CP(AY, y), CP(BY, y), CP(KY, y), h);
                    U[j] = u;
                    W[j] = w;
                    lE[j] = ca[j] * e;
                }
            }
            /* transposed curl: lambda_Hz -= Dx^h U ; lambda_Hx += Dz^h W */
#pragma omp parallel for schedule(static)
            for (ll y = 0; y < ny; ++y) {
                for (ll x = 0; x < nx; ++x) {
                    ll j = y * nx + x;
                    if (in_hz(&k, y, x)) lHz[j] -= d_xh(&k, U, y, x);
                    if (in_hx(&k, y, x)) lHx[j] += d_yh(&k, W, y, x);
                }
            }
            /* transpose of the H half-step: coefficient, filters */
#pragma omp parallel for schedule(static)
            for (ll y = 0; y < ny; ++y) {
                for (ll x = 0; x < nx; ++x) {
                    ll j = y * nx + x;
                    TZ[j] = 0.0;
                    TX[j] = 0.0;
                    if (in_hz(&k, y, x)) {
                        double q = cq[j] * lHz[j];
                        if (flag_h(&k, x, g->pml_x0, g->pml_x1))
                            q = cpml(&m_ex[j], CP(AXH, x), CP(BXH, x), CP(KXH, x), q);
                        TZ[j] = q;
                    }
                    if (in_hx(&k, y, x)) {
                        double q = cq[j] * lHx[j];
                        if (flag_h(&k, y, g->pml_y0, g->pml_y1))
                            q = cpml(&m_ez[j], CP(AYH, y), CP(BYH, y), CP(KYH, y), q);
                        TX[j] = q;
                    }
                }
            }
            /* transposed half-point derivatives: lambda_E += -Dx TZ + Dz TX */
#pragma omp parallel for schedule(static)
            for (ll y = 0; y < ny; ++y) {
                for (ll x = 0; x < nx; ++x) {
                    if (!in_e(&k, y, x)) continue;
                    ll j = y * nx + x;
                    lE[j] += -d_x(&k, TZ, y, x) + d_y(&k, TX, y, x);
                }
            }
        }
    }
done:
    free(U); free(W); free(TZ); free(TX);
#undef CP
    return rc;
}

/*
 * The whole reverse loop n = nt-1 .. 0 from a zero adjoint state
 * (orc_adjoint_range over [0, nt) on a fresh state).
 *   grad_r  [nt][S][n_rec]  dJ/dr
 *   grad_f  [nt][S][n_src]  dJ/df (output, may be NULL)
 *   snap_e, snap_c  [nt][S][ny_i][nx_i] interior snapshots from orc_forward
 *                   (may be NULL: no gradient is accumulated then)
 *   gca, gcb  [S][ny][nx]  per-shot gradients (output, overwritten; zero
 *                          outside the interior window)
 */
int orc_adjoint(const orc_geom *g, const double *ca, const double *cb, const double *cq,
                const double *cpml_arr, ll cpml_len,
                const ll *src, const ll *rec, ll nt,
                const double *grad_r, double *grad_f,
                const double *snap_e, const double *snap_c,
                double *gca, double *gcb)
{
    const ll n = g->n_shots * g->ny * g->nx;
    if (g->periodic) return -3;
    double *st = calloc((size_t)(7 * n), sizeof(double));
    if (!st) return -4;
    if (gca) memset(gca, 0, (size_t)n * sizeof(double));
    if (gcb) memset(gcb, 0, (size_t)n * sizeof(double));
    int rc = orc_adjoint_range(g, ca, cb, cq, cpml_arr, cpml_len, src, rec, grad_r, grad_f, snap_e, snap_c, 0,
                               st, st + n, st + 2 * n, st + 3 * n, st + 4 * n, st + 5 * n, st + 6 * n,
                               gca, gcb, 0, nt);
    free(st);
    return rc;
}

/* ---- shot sum ------------------------------------------------------------- */
/* grad[j] = sum over shots of grad_shot[s][j], shots in ascending order. */
void orc_shot_sum(ll n_shots, ll numel, const double *grad_shot, double *grad)
{
    for (ll j = 0; j < numel; ++j) {
        double acc = 0.0;
        for (ll s = 0; s < n_shots; ++s) acc += grad_shot[s * numel + j];
        grad[j] = acc;
    }
}

/* ---- gradients in the physical parameters ------------------------------- */
/*
 * dJ/deps_r and dJ/dsigma from dJ/dCa and dJ/dCb by the chain rule (the
 * page's convert_grad_ca_cb_to_eps_sigma computes the same quantities from
 * Ca, Cb and dt).  Written here directly from the coefficient definitions
 * with eps = EP0 eps_r and D = eps + sigma dt / 2:
 *     Ca = (eps - sigma dt / 2) / D,      Cb = dt / D,
 *     dCa/deps   =  sigma dt / D^2,       dCb/deps   = -dt / D^2,
 *     dCa/dsigma = -eps dt / D^2,         dCb/dsigma = -dt^2 / (2 D^2),
 * and d/deps_r = EP0 d/deps.  Either output may be NULL.
 */
void orc_eps_sigma_grad(ll n, const double *eps_r, const double *sigma, double dt,
                        const double *grad_ca, const double *grad_cb,
                        double *grad_eps_r, double *grad_sigma)
{
    const double ep0 = 8.8541878128e-12;
    for (ll j = 0; j < n; ++j) {
        const double eps = ep0 * eps_r[j];
        const double D = eps + 0.5 * sigma[j] * dt;
        const double D2 = D * D;
        const double dca_de = sigma[j] * dt / D2, dcb_de = -dt / D2;
        const double dca_ds = -eps * dt / D2, dcb_ds = -0.5 * dt * dt / D2;
        if (grad_eps_r) grad_eps_r[j] = ep0 * (grad_ca[j] * dca_de + grad_cb[j] * dcb_de);
        if (grad_sigma) grad_sigma[j] = grad_ca[j] * dca_ds + grad_cb[j] * dcb_ds;
    }
}

/* ---- FP8 E4M3 snapshot quantization ------------------------------------- */
/*
 * OCP FP8 E4M3 (the E4M3FN encoding): sign bit, 4 exponent bits with bias 7,
 * 3 mantissa bits; exponent field 0 holds the subnormals m/8 * 2^-6; the
 * exponent field 15 with mantissa 7 is NaN (no infinities), so the largest
 * finite value is 1.75 * 2^8 = 448.  Encoding rounds to the nearest value,
 * ties to an even mantissa, and saturates finite values beyond 448 (the
 * page's intrinsic path converts with saturation to the finite range).
 */
double orc_e4m3_decode(int code)
{
    const int sign = code & 0x80, e = (code >> 3) & 0xF, m = code & 7;
    double v;
    if (e == 0xF && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

int orc_e4m3_encode(double x)
{
    if (isnan(x)) return 0x7F;
    const int sign = signbit(x) ? 0x80 : 0;
    double a = fabs(x);
    if (a >= 448.0) return sign | 0x7E;
    if (a < ldexp(1.0, -6)) {                       /* subnormal range: steps of 2^-9 */
        const double q = nearbyint(a * 512.0);      /* ties to even (default rounding) */
        return sign | (int)q;                       /* q == 8 is the smallest normal, code 0x08 */
    }
    int k;
    (void)frexp(a, &k);                             /* a = f 2^k, f in [0.5, 1) */
    int e = k - 1;                                  /* a in [2^e, 2^(e+1)) */
    int m = (int)nearbyint((ldexp(a, -e) - 1.0) * 8.0);
    if (m == 8) { m = 0; e += 1; }
    int code = ((e + 7) << 3) | m;
    if (code > 0x7E) code = 0x7E;
    return sign | code;
}

/* x[i] <- decode(encode(float(x[i]))): the value a snapshot store keeps,
 * with the encoding decision taken on the float32 value as the kernels do. */
void orc_quantize_e4m3(ll n, double *x)
{
    for (ll i = 0; i < n; ++i) x[i] = orc_e4m3_decode(orc_e4m3_encode((double)(float)x[i]));
}
