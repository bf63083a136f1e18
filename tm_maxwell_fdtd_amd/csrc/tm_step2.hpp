// Two time steps per launch: the temporally blocked forward step kernel
// (gfx950, wave64).
//
// The single-step kernel (tm_step.hpp) moves every field through HBM once
// per time step.  Here a workgroup advances its tile by two steps, n -> n+1
// (stage A) and n+1 -> n+2 (stage B), in one pass: stage A's E^{n+1} and
// H^{n+1/2} rows feed stage B's register windows and LDS rows directly, so
// the state crosses HBM once per two steps.  The price is a halo of
// 2(2P-1) columns per side (stage A also computes E^{n+1} on stage B's halo)
// and a deeper row pipeline: stage B runs 2P rows behind stage A.
//
// Per iteration r (E^n row r enters):
//   stage A: Hx, Hz at row r-P, Ey at row r-2P+1      (forward_kernel_h/_e)
//   stage B: Hx, Hz at row r-3P, Ey at row r-4P+1     (the same, one step on)
// Three phases per iteration, separated by two barriers: (1) the Hx updates
// and the rows of E that the Hz stencils need go to LDS; (2) the Hz updates,
// whose rows the E stencils need, go to LDS; (3) the E updates.  Stage B
// reads the stage-A values of its own cell (old H, CPML memories after step
// n+1) from per-thread register rings 2P rows deep; slots are compile-time
// because the row loop is unrolled by a multiple of 2P.
//
// Sources and receivers of both steps are handled in the kernel (stage B's
// E^{n+1} must already contain the source term of step n): per shot and row
// an event table names the cells that carry sources or receivers
// (add_sources_ey, record_receivers_ey).  Every workgroup that computes a
// source cell's E^{n+1} (owner or halo) adds the same sum, so halo copies
// stay identical; only the owner records.
#pragma once

#include "tm_step.hpp"

namespace tmf {

// Per-row event tables (built on the host): for shot s and row y,
// row[s*ny + y] is -1 or an event-row k; col[k*nx + x] is -1 or an event e;
// sources of e: src[sp[e] .. sp[e+1]), receivers: rec[rp[e] .. rp[e+1]),
// both in ascending index order.
struct Events {
    const int* __restrict__ row;
    const int* __restrict__ col;
    const int* __restrict__ sp;
    const int* __restrict__ src;
    const int* __restrict__ rp;
    const int* __restrict__ rec;
    int n_src, n_rec;
};

struct Fwd2Args {
    Geo g;
    Tiling t;
    const float* __restrict__ ca;
    const float* __restrict__ cb;
    const float* __restrict__ cq;
    const float* __restrict__ cp;
    // set 0: state at time n
    const float* __restrict__ E0;
    const float* __restrict__ Hx0;
    const float* __restrict__ Hz0;
    const float* __restrict__ pez0;    // Hx-update y memory [S][by][nx]
    const float* __restrict__ pex0;    // Hz-update x memory [S][ny][bx]
    const float* __restrict__ phxz0;   // E-update y memory  [S][by][nx]
    const float* __restrict__ phzx0;   // E-update x memory  [S][ny][bx]
    // set 1: state at time n+2
    float* __restrict__ E1;
    float* __restrict__ Hx1;
    float* __restrict__ Hz1;
    float* __restrict__ pez1;
    float* __restrict__ pex1;
    float* __restrict__ phxz1;
    float* __restrict__ phzx1;
    void* __restrict__ snapA_e;        // Ey^n, curl H^n (interior window) or null
    void* __restrict__ snapA_c;
    void* __restrict__ snapB_e;        // Ey^{n+1}, curl H^{n+1}
    void* __restrict__ snapB_c;
    const float* __restrict__ fA;      // f[n]   [S][n_src] (null: no sources)
    const float* __restrict__ fB;      // f[n+1]
    float* __restrict__ rA;            // r[n]   [S][n_rec] (null: no records)
    float* __restrict__ rB;            // r[n+1]
    Events ev;
};

template <int P>
struct Strip2 {
    static constexpr int OFF = 4 * P - 2;          // thread of the first owned column
    static constexpr int W = NT - 2 * OFF;          // owned columns
};

// Sum of the source amplitudes of event e (ascending source order).
__device__ __forceinline__ float event_sources(const Events& ev, int e, const float* __restrict__ f_s)
{
    float acc = 0.0f;
    for (int q = ev.sp[e]; q < ev.sp[e + 1]; ++q) acc += f_s[ev.src[q]];
    return acc;
}

template <int P, int SNAP>
__global__ __launch_bounds__(NT) void k_fwd_step2(Fwd2Args a)
{
    constexpr int W = Strip2<P>::W, OFF = Strip2<P>::OFF;
    constexpr int D = 2;               // rows of loads in flight
    constexpr int R = 2 * P;           // depth of the stage-B rings
    constexpr int U = 8;               // unroll: a multiple of R and of D
    static_assert(U % R == 0 && U % D == 0, "unroll");
    constexpr int TY0 = 5 * P - 1;     // cyt row index of row y is y - ya + TY0
    constexpr int EV0 = 4 * P - 2;     // evt row index of row y is y - ya + EV0
    __shared__ float rowEA[NT], rowEB[NT];
    __shared__ float ringA[P][NT], ringB[P][NT];
    __shared__ float cyt[CH_MAX + 8 * P][6];
    __shared__ int evt[CH_MAX + 6 * P];

    const Geo& g = a.g;
    int s, strip, chunk;
    tile_of(a.t, s, strip, chunk);
    const int tid = threadIdx.x;
    const int nx = g.nx, ny = g.ny;
    const int xs = P + strip * W;
    const int xe = min(xs + W, nx - P + 1);
    const int ya = P + chunk * a.t.CH;
    const int yb = min(ya + a.t.CH, ny - P + 1);
    const int c = xs - OFF + tid;

    // LDS tables: CPML coefficients of rows ya-5P+1 .. yb+3P-2, event rows of
    // rows ya-4P+2 .. yb+2P-1.
    {
        const int n_ev = yb - ya + 6 * P - 2;
        const bool has_ev = a.ev.row != nullptr;
        for (int i = tid; i < n_ev; i += NT) {
            const int y = ya - EV0 + i;
            evt[i] = (has_ev && y >= 0 && y < ny) ? a.ev.row[(int64_t)s * ny + y] : -1;
        }
    }
    load_row_cpml(cyt, a.cp, g, ya - TY0, yb - ya + 8 * P - 2);   // ends with a barrier

    const bool incol = c >= 0 && c < nx;
    const bool ecol = c >= P && c <= nx - P;                       // E / Hx column
    const bool own = c >= xs && c < xe;
    const bool a_col = ecol && c >= xs - (2 * P - 1) && c < xe + 2 * P - 1;
    const bool hzA_col = tid >= P - 1 && tid <= NT - P - 1 && c >= P && c <= nx - P - 1;
    const bool hzB_col = tid >= 3 * P - 2 && tid <= NT - 3 * P && c >= P && c <= nx - P - 1;
    const bool fx_h = incol && (c < g.x0 || c >= g.hx1);
    const bool fx_e = incol && (c < g.x0 || c >= g.x1);
    const bool in_x = c >= g.x0 && c < g.x1;
    const int cc = incol ? c : 0;
    const int bxc = band_x(g, cc);

    Cpml1 cx_h{0.f, 0.f, 1.f}, cx_e{0.f, 0.f, 1.f};
    if (fx_h) cx_h = cpml_at(a.cp, g.L, AXH, c);
    if (fx_e) cx_e = cpml_at(a.cp, g.L, AX, c);

    auto hx_row = [&](int h) { return h >= P && h <= ny - P - 1; };
    auto hz_row = [&](int h) { return h >= P && h <= ny - P; };
    auto fy_h = [&](int h) { return h < g.y0 || h >= g.hy1; };
    auto fy_e = [&](int y) { return y < g.y0 || y >= g.y1; };
    auto row_own = [&](int y) { return y >= ya && y < yb; };
    // stage A computes E^{n+1} on rows ya-2P+1 .. yb+2P-2 and Hz on those rows
    auto a_row = [&](int y) { return hz_row(y) && y >= ya - 2 * P + 1 && y < yb + 2 * P - 1; };

    const int64_t so = (int64_t)s * g.slab;
    const int64_t ysh = (int64_t)s * g.by * nx, xsh = (int64_t)s * g.ny * g.bx;
    const uint32_t slab_b = (uint32_t)(g.slab * 4);
    const uint32_t yb_b = (uint32_t)((int64_t)g.by * nx * 4), xb_b = (uint32_t)((int64_t)ny * g.bx * 4);
    const RBuf bE(a.E0 + so, slab_b), bHx(a.Hx0 + so, slab_b), bHz(a.Hz0 + so, slab_b);
    const RBuf bQ(a.cq, slab_b), bCa(a.ca, slab_b), bCb(a.cb, slab_b);
    const RBuf bMez(a.pez0 + ysh, yb_b), bMex(a.pex0 + xsh, xb_b);
    const RBuf bMhxz(a.phxz0 + ysh, yb_b), bMhzx(a.phzx0 + xsh, xb_b);
    float* E1 = a.E1 + so;
    float* Hx1 = a.Hx1 + so;
    float* Hz1 = a.Hz1 + so;

    // Prefetch ring (see k_fwd_step): loads of iteration r issued at r - D.
    float fE[D], fHxA[D], fQA[D], fHzA[D], fCaA[D], fCbA[D], fQB[D], fCaB[D], fCbB[D];
    float fMez[D], fMex[D], fMhzx[D], fMhxz[D];
    auto issue = [&](int u, int r, bool live) {
        const int hA = r - P, yA = r - 2 * P + 1, hB = r - 3 * P, yB = r - 4 * P + 1;
        const bool hxA = live && ecol && hx_row(hA);
        const bool hzA = live && hzA_col && a_row(hA);
        const bool eA = live && a_col && a_row(yA);
        const bool hxB = live && own && hx_row(hB) && hB >= ya - P && hB < yb + P - 1;
        const bool hzB = live && hzB_col && hz_row(hB) && row_own(hB);
        const bool eB = live && own && row_own(yB);
        fE[u] = bE.f32(live && incol && r >= 0 && r < ny, r * nx + c);
        fHxA[u] = bHx.f32(hxA, hA * nx + c);
        fQA[u] = bQ.f32(hxA || hzA, hA * nx + c);
        fHzA[u] = bHz.f32(hzA, hA * nx + c);
        fCaA[u] = bCa.f32(eA, yA * nx + c);
        fCbA[u] = bCb.f32(eA, yA * nx + c);
        fQB[u] = bQ.f32(hxB || hzB, hB * nx + c);
        fCaB[u] = bCa.f32(eB, yB * nx + c);
        fCbB[u] = bCb.f32(eB, yB * nx + c);
        fMez[u] = bMez.f32(hxA && fy_h(hA), band_y(g, hxA && fy_h(hA) ? hA : 0) * nx + c);
        fMex[u] = bMex.f32(hzA && fx_h, hA * g.bx + bxc);
        fMhzx[u] = bMhzx.f32(eA && fx_e, yA * g.bx + bxc);
        fMhxz[u] = bMhxz.f32(eA && fy_e(yA), band_y(g, eA && fy_e(yA) ? yA : 0) * nx + c);
    };

    float ewA[2 * P], hwA[2 * P], ewB[2 * P], hwB[2 * P];
    float rHz[R], rMez[R], rMex[R], rMhzx[R], rMhxz[R];   // stage-A values for stage B
#pragma unroll
    for (int i = 0; i < 2 * P; ++i) { ewA[i] = 0.f; hwA[i] = 0.f; ewB[i] = 0.f; hwB[i] = 0.f; }
#pragma unroll
    for (int i = 0; i < R; ++i) { rHz[i] = 0.f; rMez[i] = 0.f; rMex[i] = 0.f; rMhzx[i] = 0.f; rMhxz[i] = 0.f; }

    const int r_start = ya - 2 * P + 1;
    const int r_end = yb + 4 * P - 2;
#pragma unroll
    for (int i = 1; i < 2 * P; ++i) {
        const int r = r_start - 2 * P + i;
        ewA[i] = bE.f32(incol && r >= 0 && r < ny, r * nx + c);
    }
#pragma unroll
    for (int u = 0; u < D; ++u) issue(u, r_start + u, r_start + u <= r_end);

    for (int r0 = r_start;; r0 += U) {
#pragma unroll
        for (int uu = 0; uu < U; ++uu) {
            const int r = r0 + uu;
            if (r > r_end) return;
            const int u = uu % D;          // prefetch slot
            const int k = uu % R;          // ring slot of rows hA, yA (and hB, yB)
            const int hA = r - P, yA = r - 2 * P + 1, hB = r - 3 * P, yB = r - 4 * P + 1;
            const float* cthA = cyt[hA - ya + TY0];
            const float* cteA = cyt[yA - ya + TY0];
            const float* cthB = cyt[max(hB - ya + TY0, 0)];
            const float* cteB = cyt[max(yB - ya + TY0, 0)];

            // ================= phase 1: Hx of both stages ===================
#pragma unroll
            for (int i = 0; i < 2 * P - 1; ++i) ewA[i] = ewA[i + 1];
            ewA[2 * P - 1] = fE[u];
            // stage B, row hB: old value = stage A's Hx(hB), the oldest window row
            {
                float hxn = 0.0f;
                const bool doB = own && hx_row(hB) && hB >= ya - P && hB < yb + P - 1;
                float d = g.rdy * stencil<P>([&](int q) { return ewB[P - 1 + q]; },
                                             [&](int q) { return ewB[P - q]; });
                if (fy_h(hB)) {
                    float m = rMez[k];
                    d = cpml_step(m, cthB[0], cthB[1], cthB[2], d);
                    if (doB && row_own(hB)) a.pez1[ysh + (int64_t)band_y(g, hB) * nx + c] = m;
                }
                if (doB) {
                    hxn = fmaf(-fQB[u], d, hwA[0]);
                    if (row_own(hB)) Hx1[(int64_t)hB * nx + c] = hxn;
                }
#pragma unroll
                for (int i = 0; i < 2 * P - 1; ++i) hwB[i] = hwB[i + 1];
                hwB[2 * P - 1] = hxn;
            }
            // stage A, row hA
            {
                float hxn = 0.0f;
                const bool doA = ecol && hx_row(hA);
                float d = g.rdy * stencil<P>([&](int q) { return ewA[P - 1 + q]; },
                                             [&](int q) { return ewA[P - q]; });
                if (fy_h(hA)) {
                    float m = fMez[u];
                    d = cpml_step(m, cthA[0], cthA[1], cthA[2], d);
                    rMez[k] = m;
                }
                if (doA) hxn = fmaf(-fQA[u], d, fHxA[u]);
#pragma unroll
                for (int i = 0; i < 2 * P - 1; ++i) hwA[i] = hwA[i + 1];
                hwA[2 * P - 1] = hxn;
            }
            rowEA[tid] = ewA[P - 1];               // E^n row hA
            rowEB[tid] = ewB[P - 1];               // E^{n+1} row hB
            __syncthreads();

            // ================= phase 2: Hz of both stages ===================
            if (hz_row(hB) && row_own(hB)) {       // stage B first: it reads ring slot k
                float hzn = 0.0f;
                if (hzB_col) {
                    float d = g.rdx * stencil<P>([&](int q) { return rowEB[tid + q]; },
                                                 [&](int q) { return rowEB[tid - q + 1]; });
                    if (fx_h) {
                        float m = rMex[k];
                        d = cpml_step(m, cx_h.a, cx_h.b, cx_h.ik, d);
                        if (own) a.pex1[xsh + (int64_t)hB * g.bx + bxc] = m;
                    }
                    hzn = fmaf(fQB[u], d, rHz[k]);
                    if (own) Hz1[(int64_t)hB * nx + c] = hzn;
                }
                ringB[hB % P][tid] = hzn;
            }
            if (a_row(hA)) {
                float hzn = 0.0f;
                if (hzA_col) {
                    float d = g.rdx * stencil<P>([&](int q) { return rowEA[tid + q]; },
                                                 [&](int q) { return rowEA[tid - q + 1]; });
                    if (fx_h) {
                        float m = fMex[u];
                        d = cpml_step(m, cx_h.a, cx_h.b, cx_h.ik, d);
                        rMex[k] = m;
                    }
                    hzn = fmaf(fQA[u], d, fHzA[u]);
                }
                ringA[hA % P][tid] = hzn;
                rHz[k] = hzn;
            }
            __syncthreads();

            // ================= phase 3: E of both stages ====================
            // stage B, row yB (owned cells): E^{n+2}
            if (row_own(yB)) {
                if (own) {
                    const float* hzr = ringB[yB % P];
                    float uu_ = g.rdx * stencil<P>([&](int q) { return hzr[tid + q - 1]; },
                                                   [&](int q) { return hzr[tid - q]; });
                    if (fx_e) {
                        float m = rMhzx[k];
                        uu_ = cpml_step(m, cx_e.a, cx_e.b, cx_e.ik, uu_);
                        a.phzx1[xsh + (int64_t)yB * g.bx + bxc] = m;
                    }
                    float vv = g.rdy * stencil<P>([&](int q) { return hwB[P - 1 + q]; },
                                                  [&](int q) { return hwB[P - q]; });
                    if (fy_e(yB)) {
                        float m = rMhxz[k];
                        vv = cpml_step(m, cteB[3], cteB[4], cteB[5], vv);
                        a.phxz1[ysh + (int64_t)band_y(g, yB) * nx + c] = m;
                    }
                    const float curl = uu_ - vv;
                    const float ev = ewB[0];
                    if constexpr (SNAP != SNAP_NONE) {
                        if (in_x && yB >= g.y0 && yB < g.y1) {
                            const int64_t w = ((int64_t)s * g.nyi + (yB - g.y0)) * g.nxi + (c - g.x0);
                            snap_store<SNAP>(a.snapB_e, w, ev);
                            snap_store<SNAP>(a.snapB_c, w, curl);
                        }
                    }
                    float en = fmaf(fCaB[u], ev, fCbB[u] * curl);
                    const int erow = evt[yB - ya + EV0];
                    if (erow >= 0) {
                        const int e = a.ev.col[(int64_t)erow * nx + c];
                        if (e >= 0) {
                            if (a.fB) en += event_sources(a.ev, e, a.fB + (int64_t)s * a.ev.n_src);
                            if (a.rB)
                                for (int q = a.ev.rp[e]; q < a.ev.rp[e + 1]; ++q)
                                    a.rB[(int64_t)s * a.ev.n_rec + a.ev.rec[q]] = en;
                        }
                    }
                    E1[(int64_t)yB * nx + c] = en;
                }
            }
            // stage A, row yA: E^{n+1} on stage B's whole neighbourhood
            {
                float en = 0.0f;
                if (a_row(yA) && a_col) {
                    const float* hzr = ringA[yA % P];
                    float uu_ = g.rdx * stencil<P>([&](int q) { return hzr[tid + q - 1]; },
                                                   [&](int q) { return hzr[tid - q]; });
                    if (fx_e) {
                        float m = fMhzx[u];
                        uu_ = cpml_step(m, cx_e.a, cx_e.b, cx_e.ik, uu_);
                        rMhzx[k] = m;
                    }
                    float vv = g.rdy * stencil<P>([&](int q) { return hwA[P - 1 + q]; },
                                                  [&](int q) { return hwA[P - q]; });
                    if (fy_e(yA)) {
                        float m = fMhxz[u];
                        vv = cpml_step(m, cteA[3], cteA[4], cteA[5], vv);
                        rMhxz[k] = m;
                    }
                    const float curl = uu_ - vv;
                    const float ev = ewA[0];
                    if constexpr (SNAP != SNAP_NONE) {
                        if (own && row_own(yA) && in_x && yA >= g.y0 && yA < g.y1) {
                            const int64_t w = ((int64_t)s * g.nyi + (yA - g.y0)) * g.nxi + (c - g.x0);
                            snap_store<SNAP>(a.snapA_e, w, ev);
                            snap_store<SNAP>(a.snapA_c, w, curl);
                        }
                    }
                    en = fmaf(fCaA[u], ev, fCbA[u] * curl);
                    const int erow = evt[yA - ya + EV0];
                    if (erow >= 0) {
                        const int e = a.ev.col[(int64_t)erow * nx + c];
                        if (e >= 0) {
                            if (a.fA) en += event_sources(a.ev, e, a.fA + (int64_t)s * a.ev.n_src);
                            if (a.rA && own && row_own(yA))
                                for (int q = a.ev.rp[e]; q < a.ev.rp[e + 1]; ++q)
                                    a.rA[(int64_t)s * a.ev.n_rec + a.ev.rec[q]] = en;
                        }
                    }
                }
#pragma unroll
                for (int i = 0; i < 2 * P - 1; ++i) ewB[i] = ewB[i + 1];
                ewB[2 * P - 1] = en;
            }
            issue(u, r + D, r + D <= r_end);
        }
    }
}

}  // namespace tmf
