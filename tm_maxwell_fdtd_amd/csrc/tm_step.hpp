// Fused single-pass time-step kernels of the TM FDTD forward and of its
// exact adjoint (gfx950, wave64).
//
// One launch advances every shot by one time step.  A workgroup of NT = 256
// threads owns a strip of W = NT - 4P + 2 columns and a chunk of CH rows of
// one shot and streams down the chunk one row per iteration:
//   * y-derivatives run on register windows of 2P rows per thread (each
//     thread holds one column);
//   * x-derivatives read a row staged in LDS by the whole workgroup;
//   * the H half-step of a row and the E step of the row 2P-1 above it are
//     computed in the same iteration, so H never makes a round trip through
//     HBM between the two half-steps.
// Columns within 2P-1 of the strip edges and rows within 2P-1 of the chunk
// edges are read (and their H values recomputed) but written by the
// neighbouring workgroup only.  The state is therefore double-buffered: a
// step reads set "0" and writes set "1" (fields and CPML memories).
//
// Forward step (tide-GPR 0.0.9, maxwell.cu, forward_kernel_h then
// forward_kernel_e):
//   Hx -= Cq filt_y(Dz^h Ey),  Hz += Cq filt_x(Dx^h Ey)          (H rows h)
//   Ey  = Ca Ey + Cb (filt_x(Dx Hz) - filt_y(Dz Hx))             (E rows h-P+1)
// with filt(d) = d / kappa + m, m <- b m + a d inside the CPML bands.
//
// Adjoint step, the exact transpose of the forward step (the same page's
// header comment: time-reversed, transposed operators), per cell:
//   e = lambda_E; gradients (interior); h = Cb e; u, w = band filters of h
//   (own memories, run backwards in time); lambda_Hz -= Dx^h[u];
//   lambda_Hx += Dz^h[w]; t = band filters of Cq lambda_H;
//   lambda_E = Ca e - Dx[t_z] + Dz[t_x].
// The coefficient sits at the source point of each transposed stencil and
// that point's filter comes before the stencil.
//
// Every cell of every output array has exactly one writer; there are no
// atomics.  Floating-point operations are written out explicitly (fmaf
// where a fused multiply-add is wanted) and the library is built without
// contraction, so every template instance computes bitwise the same values
// (a checkpoint replay reproduces the original forward exactly).
#pragma once

#include "tm_common.hpp"

namespace tmf {

constexpr int NT = 256;     // threads per workgroup (4 waves)
constexpr int PREFETCH = 4;     // rows of global loads in flight ahead of the computed row
constexpr int PREFETCH_ADJ = 2; // the same for the adjoint (more streams per row)
// The row loops are unrolled by a multiple of PREFETCH and PREFETCH_ADJ, so
// that every prefetch slot is a fixed register and nothing in flight is
// copied across iterations (the register windows, which only hold values
// already waited for, may rotate through copies).
constexpr int UNROLL = 4;

template <int P>
struct Strip {
    static constexpr int W = NT - 4 * P + 2;   // owned columns per strip
    static constexpr int OFF = 2 * P - 1;      // thread of the first owned column
};

// Launch geometry of the step kernels.
struct Tiling {
    int W, CH;            // owned columns per strip, owned rows per chunk
    int nstrip, nchunk;   // strips per row, chunks per column
    int nblk;             // nstrip * nchunk * S
};

// Workgroup id -> (shot, strip, chunk).  Workgroups are dealt round-robin to
// the 8 XCDs; the remap gives each XCD a contiguous range of logical ids, so
// vertically adjacent chunks (which share 2P-1 halo rows) run on the same
// XCD and meet in its L2.
__device__ __forceinline__ void tile_of(const Tiling& t, int& s, int& strip, int& chunk)
{
    const int L = blockIdx.x;
    const int q = t.nblk >> 3, rem = t.nblk & 7;
    const int xcd = L & 7, j = L >> 3;
    const int logical = xcd * q + (xcd < rem ? xcd : rem) + j;
    chunk = logical % t.nchunk;
    const int rest = logical / t.nchunk;
    strip = rest % t.nstrip;
    s = rest / t.nstrip;
}

// CPML recursion on one point: memory m <- b m + a d; returns d / kappa + m.
// (m is updated in place through the reference.)
__device__ __forceinline__ float cpml_step(float& m, float a, float b, float inv_k, float d)
{
    m = fmaf(b, m, a * d);
    return fmaf(d, inv_k, m);
}

// sum_k c_k (hi_k - lo_k), k = 1..P, accumulated in k order.
template <int P, typename Hi, typename Lo>
__device__ __forceinline__ float stencil(Hi hi, Lo lo)
{
    float acc = coef<P>(1) * (hi(1) - lo(1));
#pragma unroll
    for (int k = 2; k <= P; ++k) acc = fmaf(coef<P>(k), hi(k) - lo(k), acc);
    return acc;
}

// Inverse kappa and a, b of one CPML row of the packed [12][L] table.
struct Cpml1 {
    float a, b, ik;
};
__device__ __forceinline__ Cpml1 cpml_at(const float* __restrict__ cp, int L, int row_a, int i)
{
    // rows are ordered a, b, kappa for each of the four grids
    return Cpml1{cp[row_a * L + i], cp[(row_a + 1) * L + i], 1.0f / cp[(row_a + 2) * L + i]};
}

constexpr int CH_MAX = 256;  // largest chunk height (rows) the LDS tables hold

// Raw buffer view of one array (at most 2 GiB) for loads: a lane whose
// predicate is false gets 0 without a memory access, because its byte
// offset lies outside the buffer's range.  Loads therefore need no
// branches, which keeps the in-order vector-memory counter exact and lets
// prefetched rows stay in flight.
struct RBuf {
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ RBuf(const void* p, uint32_t bytes)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000))
    {
    }
    __device__ __forceinline__ float f32(bool ok, int idx) const
    {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, ok ? idx * 4 : OOB, 0, 0));
    }
    __device__ __forceinline__ float bf16(bool ok, int idx) const
    {
        const uint16_t h = __builtin_amdgcn_raw_buffer_load_b16(r, ok ? idx * 2 : OOB, 0, 0);
        return bf16_to_f32(h);
    }
    static constexpr int OOB = (int)0x80000000u;   // >= every buffer size (slabs are < 2 GiB)
};

// Per-row CPML coefficients of rows y_first .. y_first+n-1 into LDS:
// t[i] = {a, b, 1/kappa} of the half grid (H updates) then of the integer
// grid (E updates) for row y_first + i.  Read once per workgroup so that the
// row loop never issues a vector load outside its prefetch groups.
__device__ __forceinline__ void load_row_cpml(float (*t)[6], const float* __restrict__ cp, const Geo& g,
                                              int y_first, int n)
{
    for (int i = threadIdx.x; i < 6 * n; i += blockDim.x) {
        const int row = i / 6, k = i - 6 * row;
        const int y = y_first + row;
        const int base = k < 3 ? AYH : AY;
        const int kk = k < 3 ? k : k - 3;
        float v = 0.0f;
        if (y >= 0 && y < g.ny) {
            v = cp[(base + kk) * g.L + y];
            if (kk == 2) v = 1.0f / v;
        }
        t[row][k] = v;
    }
    __syncthreads();
}

// Unconditional load of p[idx], or of p[0] when ok is false (the caller
// ignores the value then, or p[0] is a zero halo cell).  No branch, so the
// vector-memory counter stays exact (see RBuf).
__device__ __forceinline__ float ld_or0(const float* __restrict__ p, bool ok, int idx)
{
    // unsigned 32-bit byte offset from a uniform base: one VGPR per address
    const uint32_t off = ok ? (uint32_t)idx * 4u : 0u;
    return *reinterpret_cast<const float*>(reinterpret_cast<const char*>(p) + off);
}

// ---------------------------------------------------------------------------
// Forward step
// ---------------------------------------------------------------------------
struct FwdArgs {
    Geo g;
    Tiling t;
    const float* __restrict__ ca;
    const float* __restrict__ cb;
    const float* __restrict__ cq;
    const float* __restrict__ cp;      // CPML table [12][L]
    const float* __restrict__ E0;      // state at step n (set 0)
    const float* __restrict__ Hx0;
    const float* __restrict__ Hz0;
    const float* __restrict__ pez0;    // Hx-update y memory, y bands [S][by][nx]
    const float* __restrict__ pex0;    // Hz-update x memory, x bands [S][ny][bx]
    float* __restrict__ E1;            // state at step n+1 (set 1)
    float* __restrict__ Hx1;
    float* __restrict__ Hz1;
    float* __restrict__ pez1;
    float* __restrict__ pex1;
    const float* __restrict__ phxz0;   // E-update y memory [S][by][nx]
    const float* __restrict__ phzx0;   // E-update x memory [S][ny][bx]
    float* __restrict__ phxz1;
    float* __restrict__ phzx1;
    void* __restrict__ snap_e;         // Ey^n on the interior window, or null
    void* __restrict__ snap_c;         // curl H^n on the interior window
};

template <int P, int SNAP>
__global__ __launch_bounds__(NT) void k_fwd_step(FwdArgs a)
{
    constexpr int W = Strip<P>::W, OFF = Strip<P>::OFF;
    constexpr int D = PREFETCH;
    __shared__ float rowE[NT];
    __shared__ float ring[P][NT];
    __shared__ float cyt[CH_MAX + 2 * P][6];

    const Geo& g = a.g;
    int s, strip, chunk;
    tile_of(a.t, s, strip, chunk);
    const int tid = threadIdx.x;
    const int nx = g.nx, ny = g.ny;
    const int xs = P + strip * W;
    const int xe = min(xs + W, nx - P + 1);
    const int ya = P + chunk * a.t.CH;
    const int yb = min(ya + a.t.CH, ny - P + 1);
    load_row_cpml(cyt, a.cp, g, ya - P, yb - ya + 2 * P - 1);   // rows ya-P .. yb+P-2
    const int c = xs - OFF + tid;                       // this thread's column
    const bool own = c >= xs && c < xe;
    const bool incol = c >= 0 && c < nx;
    const bool hz_col = tid >= P - 1 && tid <= NT - P - 1 && c >= P && c <= nx - P - 1;
    const bool fx_h = incol && (c < g.x0 || c >= g.hx1);   // H-update x flag
    const bool fx_e = incol && (c < g.x0 || c >= g.x1);    // E-update x flag
    const bool in_x = c >= g.x0 && c < g.x1;               // interior window column
    const int64_t so = (int64_t)s * g.slab;
    const float* E0 = a.E0 + so;
    const float* Hx0 = a.Hx0 + so;
    const float* Hz0 = a.Hz0 + so;
    float* E1 = a.E1 + so;
    float* Hx1 = a.Hx1 + so;
    float* Hz1 = a.Hz1 + so;
    const int cc = incol ? c : 0;                       // clamped column for coefficient reads
    const int bxc = band_x(g, cc);
    const int64_t ysh = (int64_t)s * g.by * nx;        // this shot's y-band memory slab
    const int64_t xsh = (int64_t)s * g.ny * g.bx;      // this shot's x-band memory slab
    const int64_t ybase = ysh + cc;                    // + band row * nx
    const int64_t xbase = xsh + bxc;                   // + row * bx

    Cpml1 cx_h{0.f, 0.f, 1.f}, cx_e{0.f, 0.f, 1.f};
    if (fx_h) cx_h = cpml_at(a.cp, g.L, AXH, c);
    if (fx_e) cx_e = cpml_at(a.cp, g.L, AX, c);

    // Row predicates of one iteration r: H row h = r - P, E row y = r - 2P + 1.
    auto hx_row = [&](int h) { return h >= P && h <= ny - P - 1; };
    auto h_own = [&](int h) { return h >= ya && h < yb; };
    auto hz_row = [&](int h) { return h_own(h) && h >= P && h <= ny - P; };
    auto fy_h = [&](int h) { return h < g.y0 || h >= g.hy1; };
    auto fy_e = [&](int y) { return y < g.y0 || y >= g.y1; };

    // Buffers of this shot's slabs.
    const uint32_t yb_b = (uint32_t)((int64_t)g.by * nx * 4), xb_b = (uint32_t)((int64_t)ny * g.bx * 4);
    const RBuf bMez(a.pez0 + ysh, yb_b), bMex(a.pex0 + xsh, xb_b);
    const RBuf bMhxz(a.phxz0 + ysh, yb_b), bMhzx(a.phzx0 + xsh, xb_b);

    // Prefetch ring: every global load of iteration r (fields, coefficients
    // and CPML memories) is issued at iteration r - D into slot
    // (r - ya) % D, so the waits of one iteration only ever target loads
    // issued D iterations earlier (the vector-memory counter is in order).
    float fE[D], fQ[D], fHx[D], fHz[D], fCa[D], fCb[D];
    float fMez[D], fMex[D], fMhxz[D], fMhzx[D];
    // ``live`` is false for rows past the end of the chunk: their loads are
    // still issued (out of range, no memory access) so that every iteration
    // issues the same number of loads.
    auto issue = [&](int u, int r, bool live) {
        const int h = r - P, y = r - 2 * P + 1;
        const int jh = h * nx + c, jy = y * nx + c;
        fE[u] = ld_or0(E0, live && r >= 0 && r < ny && incol, r * nx + c);
        fQ[u] = ld_or0(a.cq, live && incol && (hx_row(h) || h_own(h)), jh);
        const bool hx_do = live && own && hx_row(h);
        fHx[u] = ld_or0(Hx0, hx_do, jh);
        fMez[u] = bMez.f32(hx_do && fy_h(h), band_y(g, h) * nx + c);
        const bool hz_do = live && hz_col && hz_row(h);
        fHz[u] = ld_or0(Hz0, hz_do, jh);
        fMex[u] = bMex.f32(hz_do && fx_h, h * g.bx + bxc);
        const bool e_do = live && own && y >= ya && y < yb;
        fCa[u] = ld_or0(a.ca, e_do, jy);
        fCb[u] = ld_or0(a.cb, e_do, jy);
        fMhzx[u] = bMhzx.f32(e_do && fx_e, y * g.bx + bxc);
        fMhxz[u] = bMhxz.f32(e_do && fy_e(y), band_y(g, y) * nx + c);
    };

    float ew[2 * P];      // E^n rows r-2P+1 .. r
    float hw[2 * P];      // Hx^{n+1/2} rows r-3P+1 .. r-P
#pragma unroll
    for (int i = 0; i < 2 * P; ++i) hw[i] = 0.0f;
    ew[0] = 0.0f;
#pragma unroll
    for (int i = 1; i < 2 * P; ++i) {
        const int r = ya - 2 * P + i;
        ew[i] = ld_or0(E0, r >= 0 && r < ny && incol, r * nx + c);
    }
    const int r_end = yb + 2 * P - 2;
#pragma unroll
    for (int u = 0; u < D; ++u) issue(u, ya + u, ya + u <= r_end);

    // The loop ends with the kernel (return, not break), so the latch of the
    // unrolled loop only ever sees windows rotated by a full UNROLL.
    for (int r0 = ya;; r0 += UNROLL) {
#pragma unroll
        for (int uu = 0; uu < UNROLL; ++uu) {
            const int r = r0 + uu;
            if (r > r_end) return;
            const int u = uu % D;
            const int h = r - P;                       // H row of this iteration
            const int y = r - 2 * P + 1;               // E row of this iteration
            const int64_t jh = (int64_t)h * nx + cc;
            // per-row CPML coefficients (uniform: scalar loads)
            const bool hy_band = fy_h(h), ey_band = fy_e(y) && y >= ya;
            const float* cth = cyt[h - ya + P];        // half-grid row h
            const float* cte = cyt[max(y - ya + P, 0)]; // integer-grid row y (used when y >= ya)

            // --- rotate the E window
#pragma unroll
            for (int i = 0; i < 2 * P - 1; ++i) ew[i] = ew[i + 1];
            ew[2 * P - 1] = fE[u];

            // --- Hx(h, c): own columns, every H row of the window
            float hxn = 0.0f;
            if (own && hx_row(h)) {
                float d = g.rdy * stencil<P>([&](int k) { return ew[P - 1 + k]; },
                                             [&](int k) { return ew[P - k]; });
                if (hy_band) {
                    float m = fMez[u];
                    d = cpml_step(m, cth[0], cth[1], cth[2], d);
                    if (h_own(h)) a.pez1[ybase + (int64_t)band_y(g, h) * nx] = m;
                }
                hxn = fmaf(-fQ[u], d, fHx[u]);
                if (h_own(h)) Hx1[jh] = hxn;
            }
#pragma unroll
            for (int i = 0; i < 2 * P - 1; ++i) hw[i] = hw[i + 1];
            hw[2 * P - 1] = hxn;

            rowE[tid] = ew[P - 1];                     // E^n row h
            __syncthreads();

            // --- Hz(h, c): the owned rows, owned columns plus P on each side
            if (hz_row(h)) {
                float hzn = 0.0f;
                if (hz_col) {
                    float d = g.rdx * stencil<P>([&](int k) { return rowE[tid + k]; },
                                                 [&](int k) { return rowE[tid - k + 1]; });
                    if (fx_h) {
                        float m = fMex[u];
                        d = cpml_step(m, cx_h.a, cx_h.b, cx_h.ik, d);
                        if (own) a.pex1[xbase + (int64_t)h * g.bx] = m;
                    }
                    hzn = fmaf(fQ[u], d, fHz[u]);
                    if (own) Hz1[jh] = hzn;
                }
                ring[h % P][tid] = hzn;
            }
            __syncthreads();

            // --- Ey(y, c): owned cells
            if (y >= ya && own) {
                const float* hzr = ring[y % P];
                float uu_ = g.rdx * stencil<P>([&](int k) { return hzr[tid + k - 1]; },
                                               [&](int k) { return hzr[tid - k]; });
                if (fx_e) {
                    float m = fMhzx[u];
                    uu_ = cpml_step(m, cx_e.a, cx_e.b, cx_e.ik, uu_);
                    a.phzx1[xbase + (int64_t)y * g.bx] = m;
                }
                float v = g.rdy * stencil<P>([&](int k) { return hw[P - 1 + k]; },
                                             [&](int k) { return hw[P - k]; });
                if (ey_band) {
                    float m = fMhxz[u];
                    v = cpml_step(m, cte[3], cte[4], cte[5], v);
                    a.phxz1[ybase + (int64_t)band_y(g, y) * nx] = m;
                }
                const float curl = uu_ - v;
                const float ev = ew[0];
                if constexpr (SNAP != SNAP_NONE) {
                    if (in_x && y >= g.y0 && y < g.y1) {
                        const int64_t w = ((int64_t)s * g.nyi + (y - g.y0)) * g.nxi + (c - g.x0);
                        snap_store<SNAP>(a.snap_e, w, ev);
                        snap_store<SNAP>(a.snap_c, w, curl);
                    }
                }
                E1[(int64_t)y * nx + c] = fmaf(fCa[u], ev, fCb[u] * curl);
            }
            // refill this slot last, once its old values are dead
            issue(u, r + D, r + D <= r_end);
        }
    }
}

// ---------------------------------------------------------------------------
// Adjoint step
// ---------------------------------------------------------------------------
struct AdjArgs {
    Geo g;
    Tiling t;
    const float* __restrict__ ca;
    const float* __restrict__ cb;
    const float* __restrict__ cq;
    const float* __restrict__ cp;
    const float* __restrict__ lE0;     // adjoint state after step n+1 (set 0)
    const float* __restrict__ lHx0;
    const float* __restrict__ lHz0;
    const float* __restrict__ fhzx0;   // adjoint memory of the E-update x filter [S][ny][bx]
    const float* __restrict__ fhxz0;   // ... E-update y filter [S][by][nx]
    const float* __restrict__ fex0;    // ... Hz-update x filter [S][ny][bx]
    const float* __restrict__ fez0;    // ... Hx-update y filter [S][by][nx]
    float* __restrict__ lE1;           // set 1
    float* __restrict__ lHx1;
    float* __restrict__ lHz1;
    float* __restrict__ fhzx1;
    float* __restrict__ fhxz1;
    float* __restrict__ fex1;
    float* __restrict__ fez1;
    const void* __restrict__ snap_e;   // Ey^n, curl H^n of this step, or null
    const void* __restrict__ snap_c;
    float* __restrict__ gca;           // per-shot gradients [S][ny][nx], or null
    float* __restrict__ gcb;
};

template <int P, int SNAP>
__global__ __launch_bounds__(NT) void k_adj_step(AdjArgs a)
{
    constexpr int W = Strip<P>::W, OFF = Strip<P>::OFF;
    constexpr int D = PREFETCH_ADJ;
    __shared__ float rowU[NT];
    __shared__ float ring[P][NT];
    __shared__ float cyt[CH_MAX + 4 * P][6];

    const Geo& g = a.g;
    int s, strip, chunk;
    tile_of(a.t, s, strip, chunk);
    const int tid = threadIdx.x;
    const int nx = g.nx, ny = g.ny;
    const int xs = P + strip * W;
    const int xe = min(xs + W, nx - P + 1);
    const int ya = P + chunk * a.t.CH;
    const int yb = min(ya + a.t.CH, ny - P + 1);
    load_row_cpml(cyt, a.cp, g, ya - 2 * P + 1, yb - ya + 4 * P - 2);   // rows ya-2P+1 .. yb+2P-2
    const int c = xs - OFF + tid;
    const bool own = c >= xs && c < xe;
    const bool e_col = c >= P && c <= nx - P;          // E-set column
    const bool hz_col = tid >= P - 1 && tid <= NT - P - 1 && c >= P && c <= nx - P - 1;
    const bool fx_h = e_col && (c < g.x0 || c >= g.hx1);
    const bool fx_e = e_col && (c < g.x0 || c >= g.x1);
    const bool in_x = c >= g.x0 && c < g.x1;
    const int64_t so = (int64_t)s * g.slab;
    const int cc = (c >= 0 && c < nx) ? c : 0;
    const int bxc = band_x(g, cc);
    const int64_t ysh = (int64_t)s * g.by * nx, xsh = (int64_t)s * g.ny * g.bx;
    const bool grad = SNAP != SNAP_NONE && own && in_x;
    const bool do_ga = grad && a.gca != nullptr, do_gb = grad && a.gcb != nullptr;

    Cpml1 cx_h{0.f, 0.f, 1.f}, cx_e{0.f, 0.f, 1.f};
    if (fx_h) cx_h = cpml_at(a.cp, g.L, AXH, c);
    if (fx_e) cx_e = cpml_at(a.cp, g.L, AX, c);

    auto hx_row = [&](int h) { return h >= P && h <= ny - P - 1; };
    auto h_own = [&](int h) { return h >= ya && h < yb; };
    auto hz_row = [&](int h) { return h_own(h) && h >= P && h <= ny - P; };
    auto e_row = [&](int r) { return r >= P && r <= ny - P; };
    auto fy_h = [&](int h) { return h < g.y0 || h >= g.hy1; };
    auto fy_e = [&](int y) { return y < g.y0 || y >= g.y1; };
    // LDS row table: row y at index y - (ya - 2P + 1)
    auto cyrow = [&](int y) { return cyt[max(y - ya + 2 * P - 1, 0)]; };

    const uint32_t slab_b = (uint32_t)(g.slab * 4);
    const uint32_t yb_b = (uint32_t)((int64_t)g.by * nx * 4), xb_b = (uint32_t)((int64_t)ny * g.bx * 4);
    const uint32_t win = (uint32_t)((int64_t)g.nyi * g.nxi);
    const float* lE0 = a.lE0 + so;
    const float* lHx0 = a.lHx0 + so;
    const float* lHz0 = a.lHz0 + so;
    const RBuf bFhzx(a.fhzx0 + xsh, xb_b), bFhxz(a.fhxz0 + ysh, yb_b);
    const RBuf bFex(a.fex0 + xsh, xb_b), bFez(a.fez0 + ysh, yb_b);
    const int64_t wsh = (int64_t)s * win;
    const uint32_t win_b = win * (SNAP == SNAP_BF16 ? 2u : 4u);
    const RBuf bSe(SNAP == SNAP_BF16 ? (const void*)((const uint16_t*)a.snap_e + wsh) : (const void*)((const float*)a.snap_e + wsh),
                   SNAP == SNAP_NONE ? 0u : win_b);
    const RBuf bSc(SNAP == SNAP_BF16 ? (const void*)((const uint16_t*)a.snap_c + wsh) : (const void*)((const float*)a.snap_c + wsh),
                   SNAP == SNAP_NONE ? 0u : win_b);
    const RBuf bGa(a.gca + so, a.gca ? slab_b : 0u), bGb(a.gcb + so, a.gcb ? slab_b : 0u);

    // Prefetch ring (see k_fwd_step): all loads of iteration r are issued
    // at iteration r - D.
    float fE[D], fCb[D], fMx[D], fMy[D], fSe[D], fSc[D], fGa[D], fGb[D];
    float fHx[D], fQ[D], fHz[D], fMez[D], fMex[D], fCa[D];
    auto issue = [&](int u, int r, bool live) {
        const int h = r - P, y = r - 2 * P + 1;
        const int jr = r * nx + c, jh = h * nx + c, jy = y * nx + c;
        const bool e_do = live && e_col && e_row(r);
        fE[u] = ld_or0(lE0, e_do, jr);
        fCb[u] = ld_or0(a.cb, e_do, jr);
        fMx[u] = bFhzx.f32(e_do && fx_e, r * g.bx + bxc);
        fMy[u] = bFhxz.f32(e_do && fy_e(r), band_y(g, r) * nx + c);
        const bool g_do = live && r >= ya && r < yb && r >= g.y0 && r < g.y1;
        const int wi = (r - g.y0) * g.nxi + (c - g.x0);
        if constexpr (SNAP == SNAP_BF16) {
            fSe[u] = bSe.bf16(g_do && grad, wi);
            fSc[u] = bSc.bf16(g_do && grad, wi);
        } else {
            fSe[u] = bSe.f32(g_do && grad, wi);
            fSc[u] = bSc.f32(g_do && grad, wi);
        }
        fGa[u] = bGa.f32(g_do && do_ga, jr);
        fGb[u] = bGb.f32(g_do && do_gb, jr);
        const bool hx_do = live && own && hx_row(h);
        fHx[u] = ld_or0(lHx0, hx_do, jh);
        fMez[u] = bFez.f32(hx_do && fy_h(h), band_y(g, h) * nx + c);
        fQ[u] = ld_or0(a.cq, live && e_col && (hx_row(h) || h_own(h)), jh);
        const bool hz_do = live && hz_col && hz_row(h);
        fHz[u] = ld_or0(lHz0, hz_do, jh);
        fMex[u] = bFex.f32(hz_do && fx_h, h * g.bx + bxc);
        fCa[u] = ld_or0(a.ca, live && own && y >= ya && y < yb, jy);
    };

    float ed[2 * P];      // lambda_E^{n+1} rows r-2P+1 .. r
    float ww[2 * P];      // filtered Cb lambda_E for the Hx transpose, rows r-2P+1 .. r
    float ud[P + 1];      // filtered Cb lambda_E for the Hz transpose, rows r-P .. r
    float tw[2 * P];      // filtered Cq lambda_Hx, rows r-3P+1 .. r-P
#pragma unroll
    for (int i = 0; i < 2 * P; ++i) { ed[i] = 0.0f; ww[i] = 0.0f; tw[i] = 0.0f; }
#pragma unroll
    for (int i = 0; i <= P; ++i) ud[i] = 0.0f;

    // e, u, w of the E-set cell (r, c) from its loaded values; the filter
    // memories are written back on owned cells.
    auto front = [&](int r, float e, float cbv, float mx, float my, float& u, float& w) {
        const float hv = cbv * e;
        const bool r_own = own && r >= ya && r < yb && e_row(r);
        u = hv;
        if (fx_e && e_row(r)) {
            float m = mx;
            u = cpml_step(m, cx_e.a, cx_e.b, cx_e.ik, hv);
            if (r_own) a.fhzx1[xsh + (int64_t)r * g.bx + bxc] = m;
        }
        w = hv;
        if (fy_e(r) && e_col && e_row(r)) {
            const float* ct = cyrow(r);
            float m = my;
            w = cpml_step(m, ct[3], ct[4], ct[5], hv);
            if (r_own) a.fhxz1[ysh + (int64_t)band_y(g, r) * nx + c] = m;
        }
    };
    auto push = [&](float e, float u, float w) {
#pragma unroll
        for (int i = 0; i < 2 * P - 1; ++i) { ed[i] = ed[i + 1]; ww[i] = ww[i + 1]; }
        ed[2 * P - 1] = e;
        ww[2 * P - 1] = w;
#pragma unroll
        for (int i = 0; i < P; ++i) ud[i] = ud[i + 1];
        ud[P] = u;
    };

    // prologue: rows ya-2P+1 .. ya-1 (front only, no gradient)
#pragma unroll
    for (int i = 1; i < 2 * P; ++i) {
        const int r = ya - 2 * P + i;
        const bool e_do = e_col && e_row(r);
        const float e = ld_or0(lE0, e_do, r * nx + c), cbv = ld_or0(a.cb, e_do, r * nx + c);
        const float mx = bFhzx.f32(e_do && fx_e, r * g.bx + bxc);
        const float my = bFhxz.f32(e_do && fy_e(r), band_y(g, r) * nx + c);
        float u, w;
        front(r, e, cbv, mx, my, u, w);
        push(e, u, w);
    }
    const int r_end = yb + 2 * P - 2;
#pragma unroll
    for (int u = 0; u < D; ++u) issue(u, ya + u, ya + u <= r_end);

    for (int r0 = ya;; r0 += UNROLL) {
#pragma unroll
        for (int uu = 0; uu < UNROLL; ++uu) {
            const int r = r0 + uu;
            if (r > r_end) return;
            const int u = uu % D;
            {
                const float e = fE[u];
                float uv, wv;
                front(r, e, fCb[u], fMx[u], fMy[u], uv, wv);
                if constexpr (SNAP != SNAP_NONE) {
                    if (r < yb && r >= g.y0 && r < g.y1) {
                        const int64_t j = so + (int64_t)r * nx + c;
                        if (do_ga) a.gca[j] = fmaf(e, fSe[u], fGa[u]);
                        if (do_gb) a.gcb[j] = fmaf(e, fSc[u], fGb[u]);
                    }
                }
                push(e, uv, wv);
            }
            const int h = r - P;
            const int y = r - 2 * P + 1;
            const int64_t jh = so + (int64_t)h * nx + cc;
            const float q = fQ[u];

            // --- lambda_Hx(h, c) and its filtered Cq product, own columns
            float txv = 0.0f;
            if (own && hx_row(h)) {
                const float acc = stencil<P>([&](int k) { return ww[P - 1 + k]; },
                                             [&](int k) { return ww[P - k]; });
                const float lhx = fmaf(g.rdy, acc, fHx[u]);
                if (h_own(h)) a.lHx1[jh] = lhx;
                txv = q * lhx;
                if (fy_h(h)) {
                    const float* ct = cyrow(h);
                    float m = fMez[u];
                    txv = cpml_step(m, ct[0], ct[1], ct[2], txv);
                    if (h_own(h)) a.fez1[ysh + (int64_t)band_y(g, h) * nx + c] = m;
                }
            }
#pragma unroll
            for (int i = 0; i < 2 * P - 1; ++i) tw[i] = tw[i + 1];
            tw[2 * P - 1] = txv;

            rowU[tid] = ud[0];                          // u of row h
            __syncthreads();

            // --- lambda_Hz(h, c): owned rows, owned columns plus P on each side
            if (hz_row(h)) {
                float tz = 0.0f;
                if (hz_col) {
                    const float acc = stencil<P>([&](int k) { return rowU[tid + k]; },
                                                 [&](int k) { return rowU[tid - k + 1]; });
                    const float lhz = fmaf(-g.rdx, acc, fHz[u]);
                    if (own) a.lHz1[jh] = lhz;
                    tz = q * lhz;
                    if (fx_h) {
                        float m = fMex[u];
                        tz = cpml_step(m, cx_h.a, cx_h.b, cx_h.ik, tz);
                        if (own) a.fex1[xsh + (int64_t)h * g.bx + bxc] = m;
                    }
                }
                ring[h % P][tid] = tz;
            }
            __syncthreads();

            // --- lambda_E(y, c) = Ca e - Dx[t_z] + Dz[t_x]
            if (y >= ya && own) {
                const float* tzr = ring[y % P];
                const float az = stencil<P>([&](int k) { return tzr[tid + k - 1]; },
                                            [&](int k) { return tzr[tid - k]; });
                const float ay = stencil<P>([&](int k) { return tw[P - 1 + k]; },
                                            [&](int k) { return tw[P - k]; });
                a.lE1[so + (int64_t)y * nx + c] = fmaf(fCa[u], ed[0], fmaf(-az, g.rdx, ay * g.rdy));
            }
            issue(u, r + D, r + D <= r_end);
        }
    }
}

}  // namespace tmf
