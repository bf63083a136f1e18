// Resident kernels for small grids (gfx950, wave64): one workgroup holds a
// whole shot on chip and runs a run of consecutive time steps in one launch.
//
// For grids of a few thousand cells (the order-2 64x64 workload: 86 x 86
// padded, one shot) the streaming kernels are bound by launch latency and by
// the dependency chain of their row loops, not by HBM: every step costs one
// or more launches of a few microseconds.  Here a workgroup of NTS threads
// keeps the shot's fields, its band CPML memories and the per-row/column
// CPML coefficients in LDS (dynamic, up to the 160 KB of a gfx950 CU) and
// steps them with workgroup barriers only; HBM sees the initial and final
// state, the snapshots and the event rows (sources, receivers).
//
// Every cell update is the operation sequence of k_fwd_step / k_adj_step
// (same stencil helper, same fmaf placement, same filter), so results are
// bitwise those of the streaming kernels (tests compare them with one step
// per launch); only the sign of a zero may differ, where the streaming
// kernels run the identity filter on unflagged columns.
//
// Cells are dealt to threads round-robin (cell j = tid + i * NTS, CPT per
// thread), so the LDS accesses of a wave are consecutive along x.  The cell
// stencils are branch-free: every cell array has P rows and P cells of zero
// padding on each side, so every stencil read of every cell is in range, and
// values outside a field's index set are selected away (0, as the cells the
// streaming kernels never write); the compiler can then batch the LDS reads
// of all of a thread's cells.  Only the CPML filters branch, on the lanes
// of their bands.
#pragma once

#include "tm_step.hpp"

namespace tmf {

constexpr int NTS = 1024;                   // threads of a resident workgroup (16 waves)
constexpr int CPT = 8;                      // cells per thread
constexpr int SMALL_CELLS = NTS * CPT - 1;  // largest grid (ny * nx; j = ny * nx marks an unused slot)
constexpr int SMALL_MIN_SHOTS = 16;         // by default, the resident kernels run from this many shots on

struct SmallArgs {
    Geo g;
    StateLayout L;
    Model m;
    const float* __restrict__ cp;      // CPML table [12][L]
    const char* __restrict__ set0;     // state before the run (shot-major blocks)
    char* __restrict__ set1;           // state after the run
    char* __restrict__ snap;           // device snapshot store: stored step j at snap + j * snap_stride, or null
    uint64_t snap_stride;              // bytes of one stored step (all shots)
    uint32_t snap_shot_bytes;          // bytes of one shot's pairs
    int R;                             // snapshot step ratio: steps t % R == 0 are stored
    float ratio;                       // weight of a stored step's gradient term (adjoint)
    int t0, t1;                        // the run: forward t0 .. t1-1, adjoint t1-1 down to t0
    EventRows ev;                      // event rows of the run's event block
    uint32_t ev_add0, ev_out0;         // add / out row offsets of step t0
    uint32_t ev_row;                   // bytes of one step's event rows (offset increment per step)
    float* __restrict__ gca;           // per-shot gradients [S][ny][nx] (adjoint), or null
    float* __restrict__ gcb;
};

// LDS carve-up (float offsets) of the resident kernels: `ncell` padded cell
// arrays (forward: Ey, Hx, Hz; adjoint: u, w, filtered Cq lambda_Hz and
// lambda_Hx), each with `pad` floats before and after the ny*nx cells; the
// four band memories in the workspace layout ([by][nx], [ny][bx]), each
// with one spare slot at its end; the CPML coefficients [6][ny] and [6][nx]
// (a, b, 1/kappa of the half grid, then the integer grid); the event-row
// slots of the shot's rows.
struct SmallLayout {
    uint32_t pad, stride;              // padding, and floats per padded cell array
    uint32_t myh, mye, mxh, mxe;       // band memories
    uint32_t ty, tx, slot;             // tables
    uint32_t floats;                   // total
};

__host__ __device__ inline SmallLayout small_layout(const Geo& g, int ncell)
{
    SmallLayout s;
    s.pad = (uint32_t)(g.P * g.nx + g.P);
    s.stride = (uint32_t)(g.ny * g.nx) + 2u * s.pad;
    uint32_t o = (uint32_t)ncell * s.stride;
    const uint32_t byn = (uint32_t)(g.by * g.nx) + 1u, nbx = (uint32_t)(g.ny * g.bx) + 1u;
    s.myh = o; o += byn;
    s.mye = o; o += byn;
    s.mxh = o; o += nbx;
    s.mxe = o; o += nbx;
    s.ty = o; o += 6u * (uint32_t)g.ny;
    s.tx = o; o += 6u * (uint32_t)g.nx;
    s.slot = o; o += (uint32_t)g.ny;
    s.floats = o;
    return s;
}

// LDS bytes of the forward (3 cell arrays) or the adjoint (4).
__host__ __device__ inline uint32_t small_lds_bytes(const Geo& g, bool adjoint)
{
    return 4u * small_layout(g, adjoint ? 4 : 3).floats;
}

// One of a thread's cells, packed into one register: the ny*nx index j
// (14 bits), the row y (11 bits) and seven flags: in the E / Hx / Hz index
// sets, and the four filter sites apply (a set cell on the site's band).  A
// thread's unused slots (beyond the grid) pack j = ny*nx, the first word of
// the trailing padding, with every flag clear: their reads stay in range
// and their writes land in the padding, which only cells outside the index
// sets read.  The flags are computed once per launch; each step only
// extracts bits.
enum CellBit { CB_E = 25, CB_HX, CB_HZ, CB_FHY, CB_FHX, CB_FEY, CB_FEX };

template <int P>
__device__ __forceinline__ int pack_cell(int j, const Geo& g)
{
    const int nc = g.ny * g.nx;
    const bool ok = j < nc;
    const int y = ok ? j / g.nx : P, x = ok ? j - y * g.nx : P;
    const bool ecol = x >= P && x <= g.nx - P, erow = y >= P && y <= g.ny - P;
    const bool e = ok && ecol && erow;
    const bool hx = ok && ecol && y >= P && y <= g.ny - P - 1;
    const bool hz = ok && erow && x >= P && x <= g.nx - P - 1;
    const bool fhy = hx && (y < g.y0 || y >= g.hy1), fhx = hz && (x < g.x0 || x >= g.hx1);
    const bool fey = e && (y < g.y0 || y >= g.y1), fex = e && (x < g.x0 || x >= g.x1);
    return (ok ? j : nc) | (y << 14) | ((int)e << CB_E) | ((int)hx << CB_HX) | ((int)hz << CB_HZ) |
           ((int)fhy << CB_FHY) | ((int)fhx << CB_FHX) | ((int)fey << CB_FEY) | ((int)fex << CB_FEX);
}

struct Cell {
    int v;                                   // the packed word
    __device__ __forceinline__ int j() const { return v & 0x3fff; }
    __device__ __forceinline__ int y() const { return (v >> 14) & 0x7ff; }
    __device__ __forceinline__ bool bit(int b) const { return (v >> b) & 1; }
};

// A packed cell the compiler must treat as unknown at this point, so that
// no decoded form of it (LDS addresses, per-lane masks) stays alive across
// the time loop.
__device__ __forceinline__ Cell cell(int packed)
{
    asm volatile("" : "+v"(packed));
    return Cell{packed};
}

// Stage the band memories of set b0 and the tables into LDS.
__device__ __forceinline__ void small_stage(float* lds, const SmallLayout& sl, const RBuf& b0, const StateLayout& L,
                                            const Geo& g, const float* __restrict__ cp, const EventRows& ev, int s)
{
    const int byn = g.by * g.nx, nbx = g.ny * g.bx;
    for (int i = threadIdx.x; i <= byn; i += NTS) {
        lds[sl.myh + i] = b0.ld(i < byn, (uint32_t)i * 4u, L.oMyh);
        lds[sl.mye + i] = b0.ld(i < byn, (uint32_t)i * 4u, L.oMye);
    }
    for (int i = threadIdx.x; i <= nbx; i += NTS) {
        lds[sl.mxh + i] = b0.ld(i < nbx, (uint32_t)i * 4u, L.oMxh);
        lds[sl.mxe + i] = b0.ld(i < nbx, (uint32_t)i * 4u, L.oMxe);
    }
    for (int i = threadIdx.x; i < 6 * g.ny; i += NTS) {
        const int k = i / g.ny, y = i - k * g.ny;
        const int row = (k < 3 ? AYH : AY) + (k < 3 ? k : k - 3);
        const float v = cp[row * g.L + y];
        lds[sl.ty + i] = (k == 2 || k == 5) ? 1.0f / v : v;
    }
    for (int i = threadIdx.x; i < 6 * g.nx; i += NTS) {
        const int k = i / g.nx, x = i - k * g.nx;
        const int row = (k < 3 ? AXH : AX) + (k < 3 ? k : k - 3);
        const float v = cp[row * g.L + x];
        lds[sl.tx + i] = (k == 2 || k == 5) ? 1.0f / v : v;
    }
    int* slot = reinterpret_cast<int*>(lds + sl.slot);
    for (int y = threadIdx.x; y < g.ny; y += NTS) slot[y] = ev.row_slot[s * g.ny + y];
}

// Write the band memories back into set b1.
__device__ __forceinline__ void small_unstage(const float* lds, const SmallLayout& sl, const RBuf& b1,
                                              const StateLayout& L, const Geo& g)
{
    const int byn = g.by * g.nx, nbx = g.ny * g.bx;
    for (int i = threadIdx.x; i < byn; i += NTS) {
        b1.st(true, lds[sl.myh + i], (uint32_t)i * 4u, L.oMyh);
        b1.st(true, lds[sl.mye + i], (uint32_t)i * 4u, L.oMye);
    }
    for (int i = threadIdx.x; i < nbx; i += NTS) {
        b1.st(true, lds[sl.mxh + i], (uint32_t)i * 4u, L.oMxh);
        b1.st(true, lds[sl.mxe + i], (uint32_t)i * 4u, L.oMxe);
    }
}

// One filter site: the recursion on the cell's memory slot mem[idx()]
// where the site applies (coefficients tab[0], tab[n], tab[2n]), the
// identity elsewhere.  Only the lanes on the site's band touch LDS; a wave
// off every band skips the branch.
template <typename Idx>
__device__ __forceinline__ float site(bool on, float* mem, Idx idx, const float* tab, int n, float d)
{
    if (on) {
        const int i = idx();
        float m = mem[i];
        d = cpml_step(m, tab[0], tab[n], tab[2 * n], d);
        mem[i] = m;
    }
    return d;
}

// ---------------------------------------------------------------------------
// Forward: steps t0 .. t1-1 of shot blockIdx.x
// ---------------------------------------------------------------------------
template <int P, int SNAP>
__global__ __launch_bounds__(NTS) void k_fwd_small(SmallArgs a)
{
    extern __shared__ float lds[];
    const Geo& g = a.g;
    const StateLayout& L = a.L;
    const int s = blockIdx.x, tid = threadIdx.x;
    const int ny = g.ny, nx = g.nx, nc = ny * nx;
    const SmallLayout sl = small_layout(g, 3);
    float* const sE = lds + sl.pad;
    float* const sHx = sE + sl.stride;
    float* const sHz = sHx + sl.stride;
    float* const myh = lds + sl.myh;
    float* const mye = lds + sl.mye;
    float* const mxh = lds + sl.mxh;
    float* const mxe = lds + sl.mxe;
    const float* const ty = lds + sl.ty;
    const float* const tx = lds + sl.tx;
    const int* const slot = reinterpret_cast<const int*>(lds + sl.slot);

    const RBuf b0(a.set0 + (int64_t)s * L.shot_bytes, L.shot_bytes);
    const RBuf b1(a.set1 + (int64_t)s * L.shot_bytes, L.shot_bytes);
    const RBuf bm(a.m.base + (int64_t)s * a.m.shot_stride, a.m.bytes);
    const RBuf bev(a.ev.base, a.ev.bytes);

    for (int i = tid - (int)sl.pad; i < nc + (int)sl.pad; i += NTS) {
        const bool in = i >= 0 && i < nc;
        sE[i] = b0.ld(in, (uint32_t)i * 4u, L.oE);
        sHx[i] = b0.ld(in, (uint32_t)i * 4u, L.oHx);
        sHz[i] = b0.ld(in, (uint32_t)i * 4u, L.oHz);
    }
    small_stage(lds, sl, b0, L, g, a.cp, a.ev, s);

    // own cells and their coefficients
    int pk[CPT];
    float ca[CPT], cb[CPT], cq[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int j = tid + i * NTS;
        const bool ok = j < nc;
        pk[i] = pack_cell<P>(j, g);
        ca[i] = bm.ld(ok, (uint32_t)j * 4u, a.m.oCa);
        cb[i] = bm.ld(ok, (uint32_t)j * 4u, a.m.oCb);
        cq[i] = bm.ld(ok, (uint32_t)j * 4u, a.m.oCq);
    }
    __syncthreads();

    // source amplitudes of the own cells on event rows, one step ahead
    float add[CPT];
    auto load_add = [&](int tt, float (&dst)[CPT]) {
        const bool live = tt < a.t1;
        const uint32_t off = a.ev_add0 + (uint32_t)(live ? tt - a.t0 : 0) * a.ev_row;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const Cell c = cell(pk[i]);
            const int y = c.y(), gs = slot[y];
            dst[i] = bev.ld(live && c.bit(CB_E) && gs >= 0, (uint32_t)(gs * nx + c.j() - y * nx) * 4u, off);
        }
    };
    load_add(a.t0, add);

    drain_vmem();
    for (int tt = a.t0; tt < a.t1; ++tt) {
        float add_n[CPT];
        load_add(tt + 1, add_n);

        // ---- H half-step (reads Ey^n)
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const Cell c = cell(pk[i]);
            const int j = c.j();
            float dy = g.rdy * stencil<P>([&](int k) { return sE[j + k * nx]; },
                                          [&](int k) { return sE[j - (k - 1) * nx]; });
            float dx = g.rdx * stencil<P>([&](int k) { return sE[j + k]; }, [&](int k) { return sE[j - k + 1]; });
            dy = site(c.bit(CB_FHY), myh, [&] { const int y = c.y(); return band_y(g, y) * nx + (j - y * nx); },
                      ty + c.y(), ny, dy);
            dx = site(c.bit(CB_FHX), mxh, [&] { const int y = c.y(); return y * g.bx + band_x(g, j - y * nx); },
                      tx + (j - c.y() * nx), nx, dx);
            const float hx = sHx[j], hz = sHz[j];
            sHx[j] = c.bit(CB_HX) ? fmaf(-cq[i], dy, hx) : hx;
            sHz[j] = c.bit(CB_HZ) ? fmaf(cq[i], dx, hz) : hz;
        }
        __syncthreads();

        // ---- E step (reads H^{n+1/2}), snapshots, sources, receivers
        const bool stored = SNAP != SNAP_NONE && tt % a.R == 0;
        const RBuf bsp(stored ? a.snap + (uint64_t)(tt / a.R) * a.snap_stride + (uint64_t)s * a.snap_shot_bytes
                              : nullptr,
                       stored ? a.snap_shot_bytes : 0u);
        const uint32_t out_off = a.ev_out0 + (uint32_t)(tt - a.t0) * a.ev_row;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const Cell c = cell(pk[i]);
            const int j = c.j();
            float uu = g.rdx * stencil<P>([&](int k) { return sHz[j + k - 1]; }, [&](int k) { return sHz[j - k]; });
            float v = g.rdy * stencil<P>([&](int k) { return sHx[j + (k - 1) * nx]; },
                                         [&](int k) { return sHx[j - k * nx]; });
            uu = site(c.bit(CB_FEX), mxe, [&] { const int y = c.y(); return y * g.bx + band_x(g, j - y * nx); },
                      tx + 3 * nx + (j - c.y() * nx), nx, uu);
            v = site(c.bit(CB_FEY), mye, [&] { const int y = c.y(); return band_y(g, y) * nx + (j - y * nx); },
                     ty + 3 * ny + c.y(), ny, v);
            const float curl = uu - v;
            const float ev = sE[j];
            const int y = c.y(), x = j - y * nx;
            if constexpr (SNAP != SNAP_NONE) {
                const bool in_w = c.bit(CB_E) && y >= g.y0 && y < g.y1 && x >= g.x0 && x < g.x1;
                snap_put2<SNAP>(bsp, stored && in_w, (uint32_t)((y - g.y0) * g.nxi + (x - g.x0)), ev, curl);
            }
            float en = fmaf(ca[i], ev, cb[i] * curl);
            const int gs = slot[y];
            const bool evr = c.bit(CB_E) && gs >= 0;
            en = evr ? en + add[i] : en;
            bev.st(evr, en, (uint32_t)(gs * nx + x) * 4u, out_off);
            sE[j] = c.bit(CB_E) ? en : ev;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < CPT; ++i) add[i] = add_n[i];
    }

    for (int i = tid; i < nc; i += NTS) {
        b1.st(true, sE[i], (uint32_t)i * 4u, L.oE);
        b1.st(true, sHx[i], (uint32_t)i * 4u, L.oHx);
        b1.st(true, sHz[i], (uint32_t)i * 4u, L.oHz);
    }
    small_unstage(lds, sl, b1, L, g);
}

// ---------------------------------------------------------------------------
// Exact adjoint: steps t1-1 down to t0 of shot blockIdx.x
// ---------------------------------------------------------------------------
template <int P, int SNAP>
__global__ __launch_bounds__(NTS) void k_adj_small(SmallArgs a)
{
    extern __shared__ float lds[];
    const Geo& g = a.g;
    const StateLayout& L = a.L;
    const int s = blockIdx.x, tid = threadIdx.x;
    const int ny = g.ny, nx = g.nx, nc = ny * nx;
    const SmallLayout sl = small_layout(g, 4);
    float* const sU = lds + sl.pad;     // filtered Cb lambda_E for the Hz transpose (0 off the E set)
    float* const sW = sU + sl.stride;   // ... for the Hx transpose
    float* const sTZ = sW + sl.stride;  // filtered Cq lambda_Hz (0 off the Hz set)
    float* const sTX = sTZ + sl.stride; // filtered Cq lambda_Hx (0 off the Hx set)
    float* const myh = lds + sl.myh;
    float* const mye = lds + sl.mye;
    float* const mxh = lds + sl.mxh;
    float* const mxe = lds + sl.mxe;
    const float* const ty = lds + sl.ty;
    const float* const tx = lds + sl.tx;
    const int* const slot = reinterpret_cast<const int*>(lds + sl.slot);

    const RBuf b0(a.set0 + (int64_t)s * L.shot_bytes, L.shot_bytes);
    const RBuf b1(a.set1 + (int64_t)s * L.shot_bytes, L.shot_bytes);
    const RBuf bm(a.m.base + (int64_t)s * a.m.shot_stride, a.m.bytes);
    const RBuf bev(a.ev.base, a.ev.bytes);
    const uint32_t slab_b = (uint32_t)(g.slab * 4);
    const RBuf bga(a.gca + (int64_t)s * g.slab, a.gca ? slab_b : 0u);
    const RBuf bgb(a.gcb + (int64_t)s * g.slab, a.gcb ? slab_b : 0u);

    for (int i = tid; i < 4 * (int)sl.stride; i += NTS) lds[i] = 0.0f;
    small_stage(lds, sl, b0, L, g, a.cp, a.ev, s);

    auto in_window = [&](const Cell& c) {
        const int y = c.y(), x = c.j() - y * nx;
        return c.bit(CB_E) && y >= g.y0 && y < g.y1 && x >= g.x0 && x < g.x1;
    };
    // iteration i of the cell loops has work in this wave (skipping the
    // others also keeps more of the adjoint's state out of scratch)
    const int wbase = __builtin_amdgcn_readfirstlane(tid & ~63);
    auto cell_live = [&](int i) { return i * NTS + wbase < nc; };
    int pk[CPT];
    float ca[CPT], cb[CPT], cq[CPT], lE[CPT], lHx[CPT], lHz[CPT], ga[CPT], gb[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int j = tid + i * NTS;
        const bool ok = j < nc;
        pk[i] = pack_cell<P>(j, g);
        const uint32_t o = (uint32_t)j * 4u;
        ca[i] = bm.ld(ok, o, a.m.oCa);
        cb[i] = bm.ld(ok, o, a.m.oCb);
        cq[i] = bm.ld(ok, o, a.m.oCq);
        lE[i] = b0.ld(ok, o, L.oE);
        lHx[i] = b0.ld(ok, o, L.oHx);
        lHz[i] = b0.ld(ok, o, L.oHz);
        const bool gw = SNAP != SNAP_NONE && in_window(Cell{pk[i]});
        ga[i] = bga.ld(gw, o, 0u);
        gb[i] = bgb.ld(gw, o, 0u);
    }

    // residual at the receivers (add rows) and the snapshots of a step; the
    // next step's are loaded as soon as phase 1 has used this step's
    float add[CPT], se[CPT], sc[CPT];
    auto load_step = [&](int tt) {
        const bool live = tt >= a.t0;
        const uint32_t off = a.ev_add0 + (uint32_t)(live ? tt - a.t0 : 0) * a.ev_row;
        const bool stored = SNAP != SNAP_NONE && live && tt % a.R == 0;
        const RBuf bsp(stored ? a.snap + (uint64_t)(tt / a.R) * a.snap_stride + (uint64_t)s * a.snap_shot_bytes
                              : nullptr,
                       stored ? a.snap_shot_bytes : 0u);
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            add[i] = se[i] = sc[i] = 0.0f;
            if (!cell_live(i)) continue;
            const Cell c = cell(pk[i]);
            const int y = c.y(), x = c.j() - y * nx, gs = slot[y];
            add[i] = bev.ld(live && c.bit(CB_E) && gs >= 0, (uint32_t)(gs * nx + x) * 4u, off);
            const SnapPair sp = snap_get2<SNAP>(bsp, stored && in_window(c),
                                                (uint32_t)((y - g.y0) * g.nxi + (x - g.x0)));
            se[i] = sp.e;
            sc[i] = sp.c;
        }
    };
    __syncthreads();
    load_step(a.t1 - 1);

    drain_vmem();
    for (int tt = a.t1 - 1; tt >= a.t0; --tt) {
        const bool stored = SNAP != SNAP_NONE && tt % a.R == 0;
        const uint32_t out_off = a.ev_out0 + (uint32_t)(tt - a.t0) * a.ev_row;

        // ---- phase 1, transpose of the E step: residual, gradient, Cb, E-update filters
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            if (!cell_live(i)) continue;
            const Cell c = cell(pk[i]);
            const int j = c.j(), y = c.y(), x = j - y * nx;
            const bool on = c.bit(CB_E);
            const int gs = slot[y];
            const bool evr = on && gs >= 0;
            const float e = evr ? lE[i] + add[i] : lE[i];
            bev.st(evr, e, (uint32_t)(gs * nx + x) * 4u, out_off);
            if (SNAP != SNAP_NONE && stored) {
                const bool in_w = in_window(c);
                const float na = fmaf(e, se[i] * a.ratio, ga[i]), nb = fmaf(e, sc[i] * a.ratio, gb[i]);
                ga[i] = in_w ? na : ga[i];
                gb[i] = in_w ? nb : gb[i];
            }
            const float hv = cb[i] * e;
            const float u = site(c.bit(CB_FEX), mxe, [&] { return y * g.bx + band_x(g, x); }, tx + 3 * nx + x, nx, hv);
            const float w = site(c.bit(CB_FEY), mye, [&] { return band_y(g, y) * nx + x; }, ty + 3 * ny + y, ny, hv);
            sU[j] = on ? u : 0.0f;
            sW[j] = on ? w : 0.0f;
            lE[i] = e;
        }
        load_step(tt - 1);
        __syncthreads();

        // ---- phase 2, transposed curl, then Cq and the H-update filters
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            if (!cell_live(i)) continue;
            const Cell c = cell(pk[i]);
            const int j = c.j();
            const float accx = stencil<P>([&](int k) { return sW[j + k * nx]; },
                                          [&](int k) { return sW[j - (k - 1) * nx]; });
            const float accz = stencil<P>([&](int k) { return sU[j + k]; }, [&](int k) { return sU[j - k + 1]; });
            const float lhx = fmaf(g.rdy, accx, lHx[i]);
            const float lhz = fmaf(-g.rdx, accz, lHz[i]);
            const int y = c.y(), x = j - y * nx;
            const float txv = site(c.bit(CB_FHY), myh, [&] { return band_y(g, y) * nx + x; }, ty + y, ny, cq[i] * lhx);
            const float tz = site(c.bit(CB_FHX), mxh, [&] { return y * g.bx + band_x(g, x); }, tx + x, nx, cq[i] * lhz);
            const bool hx = c.bit(CB_HX), hz = c.bit(CB_HZ);
            lHx[i] = hx ? lhx : lHx[i];
            lHz[i] = hz ? lhz : lHz[i];
            sTX[j] = hx ? txv : 0.0f;
            sTZ[j] = hz ? tz : 0.0f;
        }
        __syncthreads();

        // ---- phase 3, lambda_E = Ca e - Dx[t_z] + Dz[t_x]
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            if (!cell_live(i)) continue;
            const Cell c = cell(pk[i]);
            const int j = c.j();
            const float az = stencil<P>([&](int k) { return sTZ[j + k - 1]; }, [&](int k) { return sTZ[j - k]; });
            const float ay = stencil<P>([&](int k) { return sTX[j + (k - 1) * nx]; },
                                        [&](int k) { return sTX[j - k * nx]; });
            const float en = fmaf(ca[i], lE[i], fmaf(-az, g.rdx, ay * g.rdy));
            lE[i] = c.bit(CB_E) ? en : lE[i];
        }
    }

#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int j = tid + i * NTS;
        const bool ok = j < nc;
        const uint32_t o = (uint32_t)j * 4u;
        b1.st(ok, lE[i], o, L.oE);
        b1.st(ok, lHx[i], o, L.oHx);
        b1.st(ok, lHz[i], o, L.oHz);
        const bool gw = SNAP != SNAP_NONE && in_window(Cell{pk[i]});
        bga.st(gw, ga[i], o, 0u);
        bgb.st(gw, gb[i], o, 0u);
    }
    __syncthreads();
    small_unstage(lds, sl, b1, L, g);
}

}  // namespace tmf
