// Banded resident kernels for small grids with few shots (gfx950, wave64).
//
// The single-workgroup resident kernels (tm_small.hpp) run a whole shot on
// one CU; with one or a few shots that leaves most of the device idle, and
// the streaming kernels instead pay a few microseconds of launch and
// pipeline-fill time per launch, for a few microseconds of work.  Here each
// shot is cut into bands of consecutive rows, one workgroup per band, and
// every workgroup keeps its band (plus P halo rows above and below) in LDS
// for a whole run of time steps.  After each phase whose output a
// neighbour reads through a y-stencil, the workgroup publishes its first
// and last P rows of that array to a global exchange buffer as tagged words
// and copies the neighbours' words into its halo rows once they carry the
// step's tag: two exchanges per step (forward: Hx after the H half-step, Ey
// after the E step; adjoint: the filtered w after the transposed E step,
// the filtered Cq lambda_Hx after the transposed H step).  Arrays read only
// through x-stencils need no halo.  The blocked variant at the end of this
// file steps extra rows of its neighbours instead and exchanges its whole
// state every few steps.
//
// Every cell update is the operation sequence of the single-workgroup
// resident kernels, so results are bitwise theirs (and those of the
// streaming kernels up to the sign of a zero).
//
// The workgroups of a launch wait on each other, so the runtime launches
// them cooperatively (all resident at once, or the launch fails); every
// wait is bounded: a wait that runs past spin_max polls, or sees another
// workgroup's failure, marks the launch failed (err) and every workgroup
// leaves its time loop, so the grid always drains.  Exchange rows have a
// buffer per kind and step parity: a workgroup rewrites a buffer two steps
// later, after both neighbours have published that kind for the step in
// between, which they do only after reading it.
#pragma once

#include "tm_small.hpp"

namespace tmf {

constexpr int CPTB = 4;                     // cells per thread of a band (bands are small)
constexpr int BX_WORDS = 8;                 // exchange words per thread and exchange (2 P nx <= 8 NTS)
constexpr int BX_BATCH = 2;                 // ... polled together
// Sleep units (64 clocks each) before a thread's first poll of an exchange:
// on the 300^2 order-4 4-shot grid 6 units took forward + adjoint from 33.7
// to 34.7 Gcell/s (2 units: 34.3, 4: 34.6, 8: 34.3).
constexpr int BX_POLL_WAIT = 6;

struct BandArgs {
    SmallArgs a;               // the run (as for the single-workgroup kernels)
    int rb;                    // owned rows per band (the last band: the rest, at least P)
    int nband;                 // bands per shot; workgroup w = shot * nband + band
    uint64_t* __restrict__ xbuf;  // exchange rows [workgroup][kind][parity][side: first, last][P][nx]:
                                  // (step tag << 32) | value bits; cleared before each launch
    int* __restrict__ err;        // set to 1 when a wait fails
    int spin_max;                 // polls before a wait fails (<= 0: the first wait fails)
};

// LDS carve-up (float offsets): `ncell` cell arrays of rb + 2P rows (P halo
// rows above and below the band) with pad = P*nx + P floats of zeros before
// and after; the band memories of the own rows ([rb][nx] y-band memories,
// [rb][bx] x-band memories, each with one spare slot); the CPML tables
// [6][ny] and [6][nx]; the event-row slots [ny].
struct BandLayout {
    uint32_t pad, stride;              // padding, and floats per padded cell array
    uint32_t myh, mye, mxh, mxe;       // band memories of the own rows
    uint32_t ty, tx, slot;             // tables
    uint32_t floats;                   // total
};

__host__ __device__ inline BandLayout band_layout(const Geo& g, int rb, int ncell)
{
    BandLayout s;
    s.pad = (uint32_t)(g.P * g.nx + g.P);
    s.stride = (uint32_t)((rb + 2 * g.P) * g.nx) + 2u * s.pad;
    uint32_t o = (uint32_t)ncell * s.stride;
    const uint32_t yn = (uint32_t)(rb * g.nx) + 1u, xn = (uint32_t)(rb * g.bx) + 1u;
    s.myh = o; o += yn;
    s.mye = o; o += yn;
    s.mxh = o; o += xn;
    s.mxe = o; o += xn;
    s.ty = o; o += 6u * (uint32_t)g.ny;
    s.tx = o; o += 6u * (uint32_t)g.nx;
    s.slot = o; o += (uint32_t)g.ny;
    s.floats = o;
    return s;
}

__host__ __device__ inline uint32_t band_lds_bytes(const Geo& g, int rb, bool adjoint)
{
    return 4u * band_layout(g, rb, adjoint ? 4 : 3).floats;
}

// Whether a band height fits the packed cell word (14-bit local index, the
// trailing pad included) and the thread count (CPTB cells per thread).
__host__ __device__ inline bool band_rows_ok(const Geo& g, int rb)
{
    return rb >= g.P && (rb + 3 * g.P) * g.nx + g.P < (1 << 14) && rb * g.nx <= NTS * CPTB && g.ny < 2048 &&
           2 * g.P * g.nx <= BX_WORDS * NTS;
}

// One own cell of a band, packed as in tm_small.hpp, with j the index in
// the band's cell arrays (own row y -> array row y - ya + P) and y the
// global row.  Unused slots pack the first word of the trailing padding
// with every flag clear.
template <int P>
__device__ __forceinline__ int pack_band_cell(int jo, int nrow, int ya, int rb, const Geo& g)
{
    const int nx = g.nx;
    const bool ok = jo < nrow * nx;
    const int r = ok ? jo / nx : 0;
    const int y = ya + r, x = ok ? jo - r * nx : P;
    const bool ecol = x >= P && x <= nx - P, erow = y >= P && y <= g.ny - P;
    const bool e = ok && ecol && erow;
    const bool hx = ok && ecol && y >= P && y <= g.ny - P - 1;
    const bool hz = ok && erow && x >= P && x <= nx - P - 1;
    const bool fhy = hx && (y < g.y0 || y >= g.hy1), fhx = hz && (x < g.x0 || x >= g.hx1);
    const bool fey = e && (y < g.y0 || y >= g.y1), fex = e && (x < g.x0 || x >= g.x1);
    const int j = ok ? jo + P * nx : (rb + 2 * P) * nx;
    return j | (y << 14) | ((int)e << CB_E) | ((int)hx << CB_HX) | ((int)hz << CB_HZ) | ((int)fhy << CB_FHY) |
           ((int)fhx << CB_FHX) | ((int)fey << CB_FEY) | ((int)fex << CB_FEX);
}

// Per-workgroup context of a band: its rows, buffers and the exchange.
struct Band {
    int s, b, w;                       // shot, band, workgroup
    int ya, yb, nrow;                  // own rows [ya, yb)
};

__device__ __forceinline__ Band band_of(const BandArgs& ba)
{
    Band t;
    t.w = blockIdx.x;
    t.s = t.w / ba.nband;
    t.b = t.w - t.s * ba.nband;
    t.ya = t.b * ba.rb;
    t.yb = min(t.ya + ba.rb, ba.a.g.ny);
    t.nrow = t.yb - t.ya;
    return t;
}

// Stage the band memories of the own rows and the tables into LDS.
__device__ __forceinline__ void band_stage(float* lds, const BandLayout& bl, const RBuf& b0, const StateLayout& L,
                                           const Geo& g, const float* __restrict__ cp, const EventRows& ev,
                                           const Band& t)
{
    const int nx = g.nx;
    for (int i = threadIdx.x; i < t.nrow * nx; i += NTS) {
        const int r = i / nx, x = i - r * nx, y = t.ya + r;
        const bool on = y < g.y0 || y >= g.hy1;                      // a row of the y-band arrays
        const uint32_t o = (uint32_t)((on ? band_y(g, y) : 0) * nx + x) * 4u;
        lds[bl.myh + i] = b0.ld(on, o, L.oMyh);
        lds[bl.mye + i] = b0.ld(on, o, L.oMye);
    }
    for (int i = threadIdx.x; i < t.nrow * g.bx; i += NTS) {
        const uint32_t o = (uint32_t)(t.ya * g.bx + i) * 4u;
        lds[bl.mxh + i] = b0.ld(true, o, L.oMxh);
        lds[bl.mxe + i] = b0.ld(true, o, L.oMxe);
    }
    for (int i = threadIdx.x; i < 6 * g.ny; i += NTS) {
        const int k = i / g.ny, y = i - k * g.ny;
        const int row = (k < 3 ? AYH : AY) + (k < 3 ? k : k - 3);
        const float v = cp[row * g.L + y];
        lds[bl.ty + i] = (k == 2 || k == 5) ? 1.0f / v : v;
    }
    for (int i = threadIdx.x; i < 6 * nx; i += NTS) {
        const int k = i / nx, x = i - k * nx;
        const int row = (k < 3 ? AXH : AX) + (k < 3 ? k : k - 3);
        const float v = cp[row * g.L + x];
        lds[bl.tx + i] = (k == 2 || k == 5) ? 1.0f / v : v;
    }
    int* slot = reinterpret_cast<int*>(lds + bl.slot);
    for (int y = threadIdx.x; y < g.ny; y += NTS) slot[y] = ev.row_slot[t.s * g.ny + y];
}

// Write the band memories of the own rows back into set b1.
__device__ __forceinline__ void band_unstage(const float* lds, const BandLayout& bl, const RBuf& b1,
                                             const StateLayout& L, const Geo& g, const Band& t)
{
    const int nx = g.nx;
    for (int i = threadIdx.x; i < t.nrow * nx; i += NTS) {
        const int r = i / nx, x = i - r * nx, y = t.ya + r;
        const bool on = y < g.y0 || y >= g.hy1;
        const uint32_t o = (uint32_t)((on ? band_y(g, y) : 0) * nx + x) * 4u;
        b1.st(on, lds[bl.myh + i], o, L.oMyh);
        b1.st(on, lds[bl.mye + i], o, L.oMye);
    }
    for (int i = threadIdx.x; i < t.nrow * g.bx; i += NTS) {
        const uint32_t o = (uint32_t)(t.ya * g.bx + i) * 4u;
        b1.st(true, lds[bl.mxh + i], o, L.oMxh);
        b1.st(true, lds[bl.mxe + i], o, L.oMxe);
    }
}

// Exchange n of kind `kind` (0 or 1) of array A: publish the own first and
// last P rows, then copy the two neighbours' rows into the halo rows.  Each
// published word carries its step tag n + 1 next to the value (one 64-bit
// device-coherent store, which bypasses the non-coherent caches; the
// buffers are cleared before every launch), and a reader polls each word
// until it carries the tag, so the rows need no separate counter, fence or
// barrier.  Every thread publishes its own cells (pk), whose values in A
// it wrote itself in the phase just done, so publishing needs no barrier
// either; nobody reads A's halo rows between the previous exchange's
// barrier and the one that ends this exchange.  Returns false (in every
// thread) when the launch has failed.
template <int P>
__device__ __forceinline__ bool band_exchange(const BandArgs& ba, const Band& t, float* A, int kind, int n,
                                              int* quit, const int (&pk)[CPTB])
{
    const int nx = ba.a.g.nx, tid = threadIdx.x, pn = P * nx;
    const uint64_t tag = (uint64_t)(uint32_t)(n + 1) << 32;
    uint64_t* ob = ba.xbuf + (size_t)(((t.w * 2 + kind) * 2 + (n & 1)) * 2) * pn;
#pragma unroll
    for (int i = 0; i < CPTB; ++i) {
        const Cell c = cell(pk[i]);
        const int j = c.j();
        if (j >= (P + t.nrow) * nx) continue;                 // an unused slot
        const int r = c.y() - t.ya, x = j - (r + P) * nx;     // own row r, column x
        const uint64_t w = tag | __float_as_uint(A[j]);
        if (r < P) __hip_atomic_store(&ob[r * nx + x], w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (r >= t.nrow - P)
            __hip_atomic_store(&ob[pn + (r - (t.nrow - P)) * nx + x], w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // poll: a thread's words (at most BX_WORDS: 2P rows of at most 4096 / P
    // cells) are taken BX_BATCH at a time and the words of a batch are
    // loaded together in every round, so a thread with two words waits one
    // round trip, not two
    bool bad = ba.spin_max <= 0;                              // (a host-forced failure, for tests)
    const size_t nbase = (size_t)(t.s * ba.nband) * 8 * pn;  // the shot's first workgroup
#pragma unroll 1
    for (int q0 = 0; q0 < BX_WORDS && tid + q0 * NTS < 2 * pn && !bad; q0 += BX_BATCH) {
        uint32_t pending = 0;
#pragma unroll
        for (int q = 0; q < BX_BATCH; ++q) {
            const int i = tid + (q0 + q) * NTS;
            const int side = i >= pn, nb = side ? t.b + 1 : t.b - 1;
            if (i < 2 * pn && nb >= 0 && nb < ba.nband) pending |= 1u << q;   // beyond the grid: the halo stays 0
        }
        // (a short wait before the first poll, as in the blocked kernels:
        // polls sent at once mostly arrive before the neighbours' words)
        if (q0 == 0 && pending != 0) __builtin_amdgcn_s_sleep(BX_POLL_WAIT);
#pragma unroll 1
        for (int it = 0; pending != 0; ++it) {
            uint64_t w[BX_BATCH];
#pragma unroll
            for (int q = 0; q < BX_BATCH; ++q) {
                if (!((pending >> q) & 1u)) continue;
                const int i = tid + (q0 + q) * NTS;
                const int side = i >= pn, k = i - side * pn;
                const int nb = side ? t.b + 1 : t.b - 1;
                // above: the neighbour's last rows -> halo rows [0, P); below:
                // its first rows -> halo rows [P + nrow, 2P + nrow)
                const uint64_t* ib =
                    ba.xbuf + nbase + (size_t)((((nb * 2 + kind) * 2 + (n & 1)) * 2) + (side ? 0 : 1)) * pn;
                w[q] = __hip_atomic_load(&ib[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
#pragma unroll
            for (int q = 0; q < BX_BATCH; ++q) {
                if (!((pending >> q) & 1u) || (w[q] & 0xffffffff00000000ull) != tag) continue;
                const int i = tid + (q0 + q) * NTS;
                const int side = i >= pn, k = i - side * pn;
                A[(side ? P + t.nrow : 0) * nx + k] = __uint_as_float((uint32_t)w[q]);
                pending &= ~(1u << q);
            }
            if (pending == 0) break;
            if (it >= ba.spin_max ||
                ((it & 63) == 63 && __hip_atomic_load(ba.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))) {
                bad = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    if (bad) {
        __hip_atomic_store(ba.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *quit = 1;                                            // any thread may set it; all read it below
    }
    // Every poll load has been waited for, but the compiler cannot tell on
    // all paths and would otherwise wait for all memory accesses at each
    // later write of those registers (each cell of the next phases).
    drain_vmem();
    __syncthreads();
    return *quit == 0;
}

// tt % R and tt / R of a step index that moves one step at a time, kept
// without the scalar divisions (R > 0; used only while tt >= 0).
struct StepPhase {
    int ph, idx;
    __device__ __forceinline__ void init(int tt, int R)
    {
        idx = tt / R;
        ph = tt - idx * R;
    }
    __device__ __forceinline__ void next(int R)
    {
        if (++ph == R) {
            ph = 0;
            ++idx;
        }
    }
    __device__ __forceinline__ void prev(int R)
    {
        if (--ph < 0) {
            ph = R - 1;
            --idx;
        }
    }
};

// ---------------------------------------------------------------------------
// Forward: steps t0 .. t1-1, workgroup = (shot, band)
// ---------------------------------------------------------------------------
template <int P, int SNAP>
__global__ __launch_bounds__(NTS) void k_fwd_band(BandArgs ba)
{
    extern __shared__ float lds[];
    __shared__ int quit;
    const SmallArgs& a = ba.a;
    const Geo& g = a.g;
    const StateLayout& L = a.L;
    const Band t = band_of(ba);
    const int s = t.s, tid = threadIdx.x;
    const int ny = g.ny, nx = g.nx;
    const BandLayout bl = band_layout(g, ba.rb, 3);
    float* const sE = lds + bl.pad;
    float* const sHx = sE + bl.stride;
    float* const sHz = sHx + bl.stride;
    float* const myh = lds + bl.myh;
    float* const mye = lds + bl.mye;
    float* const mxh = lds + bl.mxh;
    float* const mxe = lds + bl.mxe;
    const float* const ty = lds + bl.ty;
    const float* const tx = lds + bl.tx;
    const int* const slot = reinterpret_cast<const int*>(lds + bl.slot);
    const int y_arr = t.ya - P;                    // global row of array row 0

    const RBuf b0(a.set0 + (int64_t)s * L.shot_bytes, L.shot_bytes);
    const RBuf b1(a.set1 + (int64_t)s * L.shot_bytes, L.shot_bytes);
    const RBuf bm(a.m.base + (int64_t)s * a.m.shot_stride, a.m.bytes);
    const RBuf bev(a.ev.base, a.ev.bytes);

    // fields of the array rows (own and halo; 0 off the grid) and padding
    const int arr = (ba.rb + 2 * P) * nx;
    for (int i = tid - (int)bl.pad; i < arr + (int)bl.pad; i += NTS) {
        const int gj = y_arr * nx + i;
        const bool in = i >= 0 && i < arr && gj >= 0 && gj < ny * nx;
        const uint32_t o = (uint32_t)(in ? gj : 0) * 4u;
        sE[i] = b0.ld(in, o, L.oE);
        sHx[i] = b0.ld(in, o, L.oHx);
        sHz[i] = b0.ld(in, o, L.oHz);
    }
    band_stage(lds, bl, b0, L, g, a.cp, a.ev, t);
    if (tid == 0) quit = 0;

    // iteration i of the cell loops has work in this wave
    const int wbase = __builtin_amdgcn_readfirstlane(tid & ~63), ncel = t.nrow * nx;
    auto cell_live = [&](int i) { return i * NTS + wbase < ncel; };
    int pk[CPTB];
    float ca[CPTB], cb[CPTB], cq[CPTB];
#pragma unroll
    for (int i = 0; i < CPTB; ++i) {
        const int jo = tid + i * NTS;
        const bool ok = jo < t.nrow * nx;
        pk[i] = pack_band_cell<P>(jo, t.nrow, t.ya, ba.rb, g);
        const uint32_t o = (uint32_t)(ok ? t.ya * nx + jo : 0) * 4u;
        ca[i] = bm.ld(ok, o, a.m.oCa);
        cb[i] = bm.ld(ok, o, a.m.oCb);
        cq[i] = bm.ld(ok, o, a.m.oCq);
    }
    __syncthreads();

    auto xof = [&](const Cell& c) { return c.j() - (c.y() - y_arr) * nx; };
    // source amplitudes of the cells on event rows: two steps ahead, in two
    // sets (steps of even and odd offset from t0), each reloaded right after
    // its step has used it
    auto load_add = [&](int tt, float (&dst)[CPTB]) {
        const bool in_run = tt < a.t1;
        const uint32_t off = a.ev_add0 + (uint32_t)(in_run ? tt - a.t0 : 0) * a.ev_row;
#pragma unroll
        for (int i = 0; i < CPTB; ++i) {
            dst[i] = 0.0f;
            if (!cell_live(i)) continue;
            const Cell c = cell(pk[i]);
            const int y = c.y(), gs = slot[y];
            dst[i] = bev.ld(in_run && c.bit(CB_E) && gs >= 0, (uint32_t)(gs * nx + xof(c)) * 4u, off);
        }
    };
    float add0[CPTB], add1[CPTB];
    load_add(a.t0, add0);
    load_add(a.t0 + 1, add1);

    StepPhase sp;                           // of the step
    if constexpr (SNAP != SNAP_NONE) sp.init(a.t0, a.R);
    // one step; false when the launch has failed
    auto step = [&](int tt, float (&add)[CPTB]) -> bool {
        // ---- H half-step (reads Ey^n, own rows and halo)
#pragma unroll
        for (int i = 0; i < CPTB; ++i) {
            if (!cell_live(i)) continue;
            const Cell c = cell(pk[i]);
            const int j = c.j();
            float dy = g.rdy * stencil<P>([&](int k) { return sE[j + k * nx]; },
                                          [&](int k) { return sE[j - (k - 1) * nx]; });
            float dx = g.rdx * stencil<P>([&](int k) { return sE[j + k]; }, [&](int k) { return sE[j - k + 1]; });
            dy = site(c.bit(CB_FHY), myh, [&] { return (c.y() - t.ya) * nx + xof(c); }, ty + c.y(), ny, dy);
            dx = site(c.bit(CB_FHX), mxh, [&] { return (c.y() - t.ya) * g.bx + band_x(g, xof(c)); },
                      tx + xof(c), nx, dx);
            const float hx = sHx[j], hz = sHz[j];
            sHx[j] = c.bit(CB_HX) ? fmaf(-cq[i], dy, hx) : hx;
            sHz[j] = c.bit(CB_HZ) ? fmaf(cq[i], dx, hz) : hz;
        }
        if (!band_exchange<P>(ba, t, sHx, 0, tt - a.t0, &quit, pk)) return false;

        // ---- E step (reads H^{n+1/2}), snapshots, sources, receivers
        const bool stored = SNAP != SNAP_NONE && sp.ph == 0;
        const RBuf bsp(stored ? a.snap + (uint64_t)sp.idx * a.snap_stride + (uint64_t)s * a.snap_shot_bytes
                              : nullptr,
                       stored ? a.snap_shot_bytes : 0u);
        if constexpr (SNAP != SNAP_NONE) sp.next(a.R);
        const uint32_t out_off = a.ev_out0 + (uint32_t)(tt - a.t0) * a.ev_row;
        const bool next_in = tt + 2 < a.t1;
        const uint32_t next_off = a.ev_add0 + (uint32_t)(next_in ? tt + 2 - a.t0 : 0) * a.ev_row;
#pragma unroll
        for (int i = 0; i < CPTB; ++i) {
            if (!cell_live(i)) continue;
            const Cell c = cell(pk[i]);
            const int j = c.j();
            float uu = g.rdx * stencil<P>([&](int k) { return sHz[j + k - 1]; }, [&](int k) { return sHz[j - k]; });
            float v = g.rdy * stencil<P>([&](int k) { return sHx[j + (k - 1) * nx]; },
                                         [&](int k) { return sHx[j - k * nx]; });
            uu = site(c.bit(CB_FEX), mxe, [&] { return (c.y() - t.ya) * g.bx + band_x(g, xof(c)); },
                      tx + 3 * nx + xof(c), nx, uu);
            v = site(c.bit(CB_FEY), mye, [&] { return (c.y() - t.ya) * nx + xof(c); }, ty + 3 * ny + c.y(), ny, v);
            const float curl = uu - v;
            const float ev = sE[j];
            const int y = c.y(), x = xof(c);
            if constexpr (SNAP != SNAP_NONE) {
                const bool in_w = c.bit(CB_E) && y >= g.y0 && y < g.y1 && x >= g.x0 && x < g.x1;
                snap_put2<SNAP>(bsp, stored && in_w, (uint32_t)((y - g.y0) * g.nxi + (x - g.x0)), ev, curl);
            }
            float en = fmaf(ca[i], ev, cb[i] * curl);
            const int gs = slot[y];
            const bool evr = c.bit(CB_E) && gs >= 0;
            en = evr ? en + add[i] : en;
            bev.st(evr, en, (uint32_t)(gs * nx + x) * 4u, out_off);
            add[i] = bev.ld(next_in && evr, (uint32_t)(gs * nx + x) * 4u, next_off);   // step tt + 2
            sE[j] = c.bit(CB_E) ? en : ev;
        }
        return band_exchange<P>(ba, t, sE, 1, tt - a.t0, &quit, pk);
    };
    drain_vmem();
    for (int tt = a.t0; tt < a.t1; tt += 2) {
        if (!step(tt, add0)) break;
        if (tt + 1 < a.t1 && !step(tt + 1, add1)) break;
    }


    // own rows back
    for (int i = tid; i < t.nrow * nx; i += NTS) {
        const uint32_t o = (uint32_t)(t.ya * nx + i) * 4u;
        b1.st(true, sE[P * nx + i], o, L.oE);
        b1.st(true, sHx[P * nx + i], o, L.oHx);
        b1.st(true, sHz[P * nx + i], o, L.oHz);
    }
    band_unstage(lds, bl, b1, L, g, t);
}

// ---------------------------------------------------------------------------
// Exact adjoint: steps t1-1 down to t0, workgroup = (shot, band)
// ---------------------------------------------------------------------------
template <int P, int SNAP>
__global__ __launch_bounds__(NTS) void k_adj_band(BandArgs ba)
{
    extern __shared__ float lds[];
    __shared__ int quit;
    const SmallArgs& a = ba.a;
    const Geo& g = a.g;
    const StateLayout& L = a.L;
    const Band t = band_of(ba);
    const int s = t.s, tid = threadIdx.x;
    const int ny = g.ny, nx = g.nx;
    const BandLayout bl = band_layout(g, ba.rb, 4);
    float* const sU = lds + bl.pad;     // filtered Cb lambda_E for the Hz transpose (0 off the E set)
    float* const sW = sU + bl.stride;   // ... for the Hx transpose (exchanged)
    float* const sTZ = sW + bl.stride;  // filtered Cq lambda_Hz (0 off the Hz set)
    float* const sTX = sTZ + bl.stride; // filtered Cq lambda_Hx (0 off the Hx set; exchanged)
    float* const myh = lds + bl.myh;
    float* const mye = lds + bl.mye;
    float* const mxh = lds + bl.mxh;
    float* const mxe = lds + bl.mxe;
    const float* const ty = lds + bl.ty;
    const float* const tx = lds + bl.tx;
    const int* const slot = reinterpret_cast<const int*>(lds + bl.slot);
    const int y_arr = t.ya - P;

    const RBuf b0(a.set0 + (int64_t)s * L.shot_bytes, L.shot_bytes);
    const RBuf b1(a.set1 + (int64_t)s * L.shot_bytes, L.shot_bytes);
    const RBuf bm(a.m.base + (int64_t)s * a.m.shot_stride, a.m.bytes);
    const RBuf bev(a.ev.base, a.ev.bytes);
    const uint32_t slab_b = (uint32_t)(g.slab * 4);
    const RBuf bga(a.gca + (int64_t)s * g.slab, a.gca ? slab_b : 0u);
    const RBuf bgb(a.gcb + (int64_t)s * g.slab, a.gcb ? slab_b : 0u);

    for (int i = tid; i < 4 * (int)bl.stride; i += NTS) lds[i] = 0.0f;
    band_stage(lds, bl, b0, L, g, a.cp, a.ev, t);
    if (tid == 0) quit = 0;

    auto xof = [&](const Cell& c) { return c.j() - (c.y() - y_arr) * nx; };
    auto in_window = [&](const Cell& c) {
        const int y = c.y(), x = xof(c);
        return c.bit(CB_E) && y >= g.y0 && y < g.y1 && x >= g.x0 && x < g.x1;
    };
    // iteration i of the cell loops has work in this wave
    const int wbase = __builtin_amdgcn_readfirstlane(tid & ~63), ncel = t.nrow * nx;
    auto cell_live = [&](int i) { return i * NTS + wbase < ncel; };
    int pk[CPTB];
    float ca[CPTB], cb[CPTB], cq[CPTB], lE[CPTB], lHx[CPTB], lHz[CPTB], ga[CPTB], gb[CPTB];
#pragma unroll
    for (int i = 0; i < CPTB; ++i) {
        const int jo = tid + i * NTS;
        const bool ok = jo < t.nrow * nx;
        pk[i] = pack_band_cell<P>(jo, t.nrow, t.ya, ba.rb, g);
        const uint32_t o = (uint32_t)(ok ? t.ya * nx + jo : 0) * 4u;
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

    float add[CPTB], se[CPTB], sc[CPTB];
    StepPhase lp;                           // of the step load_step reads (one lower at each call)
    if constexpr (SNAP != SNAP_NONE) lp.init(a.t1 - 1, a.R);
    auto load_step = [&](int tt) {
        const bool in_run = tt >= a.t0;
        const uint32_t off = a.ev_add0 + (uint32_t)(in_run ? tt - a.t0 : 0) * a.ev_row;
        const bool stored = SNAP != SNAP_NONE && in_run && lp.ph == 0;
        const RBuf bsp(stored ? a.snap + (uint64_t)lp.idx * a.snap_stride + (uint64_t)s * a.snap_shot_bytes
                              : nullptr,
                       stored ? a.snap_shot_bytes : 0u);
        if constexpr (SNAP != SNAP_NONE) lp.prev(a.R);
#pragma unroll
        for (int i = 0; i < CPTB; ++i) {
            add[i] = se[i] = sc[i] = 0.0f;
            if (!cell_live(i)) continue;
            const Cell c = cell(pk[i]);
            const int y = c.y(), x = xof(c), gs = slot[y];
            add[i] = bev.ld(in_run && c.bit(CB_E) && gs >= 0, (uint32_t)(gs * nx + x) * 4u, off);
            const SnapPair sp = snap_get2<SNAP>(bsp, stored && in_window(c),
                                                (uint32_t)((y - g.y0) * g.nxi + (x - g.x0)));
            se[i] = sp.e;
            sc[i] = sp.c;
        }
    };
    __syncthreads();
    load_step(a.t1 - 1);

    drain_vmem();
    StepPhase sp;                           // of the step
    if constexpr (SNAP != SNAP_NONE) sp.init(a.t1 - 1, a.R);
    for (int tt = a.t1 - 1; tt >= a.t0; --tt) {
        const bool stored = SNAP != SNAP_NONE && sp.ph == 0;
        if constexpr (SNAP != SNAP_NONE) sp.prev(a.R);
        const uint32_t out_off = a.ev_out0 + (uint32_t)(tt - a.t0) * a.ev_row;
        const int n = a.t1 - 1 - tt;

        // ---- phase 1, transpose of the E step: residual, gradient, Cb, E-update filters
#pragma unroll
        for (int i = 0; i < CPTB; ++i) {
            if (!cell_live(i)) continue;
            const Cell c = cell(pk[i]);
            const int j = c.j(), y = c.y(), x = xof(c);
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
            const float u = site(c.bit(CB_FEX), mxe, [&] { return (y - t.ya) * g.bx + band_x(g, x); },
                                 tx + 3 * nx + x, nx, hv);
            const float w = site(c.bit(CB_FEY), mye, [&] { return (y - t.ya) * nx + x; }, ty + 3 * ny + y, ny, hv);
            sU[j] = on ? u : 0.0f;
            sW[j] = on ? w : 0.0f;
            lE[i] = e;
        }
        load_step(tt - 1);
        if (!band_exchange<P>(ba, t, sW, 0, n, &quit, pk)) break;

        // ---- phase 2, transposed curl, then Cq and the H-update filters
#pragma unroll
        for (int i = 0; i < CPTB; ++i) {
            if (!cell_live(i)) continue;
            const Cell c = cell(pk[i]);
            const int j = c.j();
            const float accx = stencil<P>([&](int k) { return sW[j + k * nx]; },
                                          [&](int k) { return sW[j - (k - 1) * nx]; });
            const float accz = stencil<P>([&](int k) { return sU[j + k]; }, [&](int k) { return sU[j - k + 1]; });
            const float lhx = fmaf(g.rdy, accx, lHx[i]);
            const float lhz = fmaf(-g.rdx, accz, lHz[i]);
            const int y = c.y(), x = xof(c);
            const float txv = site(c.bit(CB_FHY), myh, [&] { return (y - t.ya) * nx + x; }, ty + y, ny, cq[i] * lhx);
            const float tz = site(c.bit(CB_FHX), mxh, [&] { return (y - t.ya) * g.bx + band_x(g, x); }, tx + x, nx,
                                  cq[i] * lhz);
            const bool hx = c.bit(CB_HX), hz = c.bit(CB_HZ);
            lHx[i] = hx ? lhx : lHx[i];
            lHz[i] = hz ? lhz : lHz[i];
            sTX[j] = hx ? txv : 0.0f;
            sTZ[j] = hz ? tz : 0.0f;
        }
        if (!band_exchange<P>(ba, t, sTX, 1, n, &quit, pk)) break;

        // ---- phase 3, lambda_E = Ca e - Dx[t_z] + Dz[t_x]
#pragma unroll
        for (int i = 0; i < CPTB; ++i) {
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
    for (int i = 0; i < CPTB; ++i) {
        const int jo = tid + i * NTS;
        const bool ok = jo < t.nrow * nx;
        const uint32_t o = (uint32_t)(ok ? t.ya * nx + jo : 0) * 4u;
        b1.st(ok, lE[i], o, L.oE);
        b1.st(ok, lHx[i], o, L.oHx);
        b1.st(ok, lHz[i], o, L.oHz);
        const bool gw = SNAP != SNAP_NONE && in_window(Cell{pk[i]});
        bga.st(gw, ga[i], o, 0u);
        bgb.st(gw, gb[i], o, 0u);
    }
    __syncthreads();
    band_unstage(lds, bl, b1, L, g, t);
}

}  // namespace tmf

namespace tmf {

// ---------------------------------------------------------------------------
// Blocked variant: one exchange per kx steps.
//
// Each workgroup computes every step on its band widened by hd = kx (2P-1)
// rows on each side (its "extended" rows), as if the extended rows were the
// whole grid.  A row's value after a step depends on rows at most 2P-1 away
// before it, so after kx steps the own rows are exact although the outer
// extended rows were computed from rows the workgroup does not hold; then
// the whole state of the extended rows outside the band (fields and band
// memories, seven words per cell) is replaced by the neighbours' own rows,
// which are exact.  Sources and receiver residuals are injected on every
// extended row, so the rows that matter are computed exactly; records,
// snapshots, source gradients and model gradients are written for the own
// rows only.  The band memories live in the cells' registers.  Exchange
// words are tagged with the exchange number, as above, and laid out so that
// a wave's lanes store and poll consecutive words; an exchange takes no
// barrier of its own (the kernels say why).
// ---------------------------------------------------------------------------

constexpr int BK_NW = 7;                    // exchanged words per cell
constexpr int CPTK = 2;                     // most cells per thread (a band's extended rows: at most 2048 cells)

struct BandKArgs {
    SmallArgs a;
    int rb, nband;                          // owned rows per band (each band at least hd), bands per shot
    int hd, kx;                             // extended rows on each side, steps between exchanges
    uint64_t* __restrict__ xbuf;            // [workgroup][parity][side][BK_NW][hd][nx] tagged words
    int* __restrict__ err;
    int spin_max;
};

struct BandKLayout {
    uint32_t pad, stride;                   // padding, and floats per padded cell array
    uint32_t ty, tx, slot;                  // tables
    uint32_t floats;
};

__host__ __device__ inline BandKLayout bandk_layout(const Geo& g, int rb, int hd, int ncell)
{
    BandKLayout s;
    s.pad = (uint32_t)(g.P * g.nx + g.P);
    s.stride = (uint32_t)((rb + 2 * hd) * g.nx) + 2u * s.pad;
    uint32_t o = (uint32_t)ncell * s.stride;
    s.ty = o; o += 6u * (uint32_t)g.ny;
    s.tx = o; o += 6u * (uint32_t)g.nx;
    s.slot = o; o += (uint32_t)g.ny;
    s.floats = o;
    return s;
}

__host__ __device__ inline uint32_t bandk_lds_bytes(const Geo& g, int rb, int hd, bool adjoint)
{
    return 4u * bandk_layout(g, rb, hd, adjoint ? 4 : 3).floats;
}

// Cells of a band's extended rows that some update can touch (columns
// P .. nx-P; bandk_cells takes the rows too).
__host__ __device__ inline int bandk_row_cells(const Geo& g, int rb, int hd)
{
    return (rb + 2 * hd) * (g.nx - 2 * g.P + 1);
}

__host__ __device__ inline bool bandk_rows_ok(const Geo& g, int rb, int hd)
{
    return rb >= hd && hd >= 2 * g.P - 1 && (rb + 2 * hd + g.P) * g.nx + g.P < (1 << 14) &&
           bandk_row_cells(g, rb, hd) <= NTS * CPTK && g.ny < 2048;
}

// Cells per thread of the kernel instance that runs a layout: 1 where the
// extended rows have at most NTS cells (half the cell registers, which the
// order-2 adjoint needs to stay out of scratch), else CPTK.
__host__ __device__ inline int bandk_cells_per_thread(const Geo& g, int rb, int hd)
{
    return bandk_row_cells(g, rb, hd) <= NTS ? 1 : CPTK;
}

// Threads of a blocked launch: with one cell per thread, one per cell that
// some update touches (rounded up to whole waves: a band's extended rows
// within rows P .. ny-P, columns P .. nx-P), so that no wave only keeps
// time at the barriers; else NTS.
__host__ __device__ inline int bandk_threads(const Geo& g, int rb, int hd)
{
    if (bandk_cells_per_thread(g, rb, hd) != 1) return NTS;
    return (bandk_row_cells(g, rb, hd) + 63) / 64 * 64;
}

struct BandK {
    int s, b, w;
    int ya, yb, nrow;                       // own rows [ya, yb)
    int ea, eb;                             // extended rows in the grid [ea, eb)
    int y_arr;                              // global row of array row 0 (ya - hd)
};

__device__ __forceinline__ BandK bandk_of(const BandKArgs& ba)
{
    BandK t;
    t.w = blockIdx.x;
    t.s = t.w / ba.nband;
    t.b = t.w - t.s * ba.nband;
    t.ya = t.b * ba.rb;
    t.yb = min(t.ya + ba.rb, ba.a.g.ny);
    t.nrow = t.yb - t.ya;
    t.ea = max(t.ya - ba.hd, 0);
    t.eb = min(t.yb + ba.hd, ba.a.g.ny);
    t.y_arr = t.ya - ba.hd;
    return t;
}

// The cells of the extended rows that some update touches: rows [ca, cb)
// of the grid's rows P .. ny-P, columns P .. nx-P (ncol of them).  The
// others (the outermost rows and columns) are never written by any update,
// so the kernels leave them as loaded (0) and neither step nor exchange
// them: on the 86^2 order-2 grid that brings a band's 6 x 86 cells to 510,
// eight waves instead of nine.
struct BandKCells {
    int ca, cb, ncol, n;
};
__device__ __forceinline__ BandKCells bandk_cells(const BandK& t, const Geo& g)
{
    BandKCells c;
    c.ca = max(t.ea, g.P);
    c.cb = min(t.eb, g.ny - g.P + 1);
    c.ncol = g.nx - 2 * g.P + 1;
    c.n = c.cb > c.ca ? (c.cb - c.ca) * c.ncol : 0;
    return c;
}

// A packed cell in a step loop: at order 2 decoded where the compiler likes
// (it keeps the decoded fields in registers across the time loop), at
// higher orders rebuilt at each use (cell(), tm_small.hpp), since their
// larger stencils leave no registers for that.
template <int P>
__device__ __forceinline__ Cell bcell(int packed)
{
    if constexpr (P == 1) return Cell{packed};
    else return cell(packed);
}

// Cell je of those (row-major from row ca, column P), packed as in
// tm_small.hpp with j its index in the cell arrays (array row y - y_arr).
template <int P>
__device__ __forceinline__ int pack_bandk_cell(int je, const BandK& t, const BandKCells& cs, int rows, const Geo& g)
{
    const int nx = g.nx;
    const bool ok = je < cs.n;
    const int r = ok ? je / cs.ncol : 0;
    const int y = ok ? cs.ca + r : t.ea, x = ok ? P + je - r * cs.ncol : P;
    const bool ecol = x >= P && x <= nx - P, erow = y >= P && y <= g.ny - P;
    const bool e = ok && ecol && erow;
    const bool hx = ok && ecol && y >= P && y <= g.ny - P - 1;
    const bool hz = ok && erow && x >= P && x <= nx - P - 1;
    const bool fhy = hx && (y < g.y0 || y >= g.hy1), fhx = hz && (x < g.x0 || x >= g.hx1);
    const bool fey = e && (y < g.y0 || y >= g.y1), fex = e && (x < g.x0 || x >= g.x1);
    const int j = ok ? (y - t.y_arr) * nx + x : rows * nx;
    return j | (y << 14) | ((int)e << CB_E) | ((int)hx << CB_HX) | ((int)hz << CB_HZ) | ((int)fhy << CB_FHY) |
           ((int)fhx << CB_FHX) | ((int)fey << CB_FEY) | ((int)fex << CB_FEX);
}

// The CPML tables and event-row slots into LDS.
__device__ __forceinline__ void bandk_tables(float* lds, const BandKLayout& bl, const Geo& g,
                                             const float* __restrict__ cp, const EventRows& ev, int s, int nth)
{
    for (int i = threadIdx.x; i < 6 * g.ny; i += nth) {
        const int k = i / g.ny, y = i - k * g.ny;
        const int row = (k < 3 ? AYH : AY) + (k < 3 ? k : k - 3);
        const float v = cp[row * g.L + y];
        lds[bl.ty + i] = (k == 2 || k == 5) ? 1.0f / v : v;
    }
    for (int i = threadIdx.x; i < 6 * g.nx; i += nth) {
        const int k = i / g.nx, x = i - k * g.nx;
        const int row = (k < 3 ? AXH : AX) + (k < 3 ? k : k - 3);
        const float v = cp[row * g.L + x];
        lds[bl.tx + i] = (k == 2 || k == 5) ? 1.0f / v : v;
    }
    int* slot = reinterpret_cast<int*>(lds + bl.slot);
    for (int y = threadIdx.x; y < g.ny; y += nth) slot[y] = ev.row_slot[s * g.ny + y];
}

// The band memories of a cell, from / to set b: every cell of a row of the
// y-band arrays has a y-memory word, every cell of a column of the x-band
// arrays an x-memory word (also where no filter site applies: those words
// pass through unchanged); 0 elsewhere.
struct CellMem {
    float yh, xh, ye, xe;
};

__device__ __forceinline__ CellMem bandk_mem_load(const RBuf& b, const StateLayout& L, const Geo& g, int y, int x,
                                                  bool ok)
{
    const bool ry = ok && flag_hy(g, y), rx = ok && flag_hx(g, x);
    const uint32_t oy = (uint32_t)((ry ? band_y(g, y) : 0) * g.nx + x) * 4u;
    const uint32_t ox = (uint32_t)(y * g.bx + (rx ? band_x(g, x) : 0)) * 4u;
    CellMem m;
    m.yh = b.ld(ry, oy, L.oMyh);
    m.ye = b.ld(ry, oy, L.oMye);
    m.xh = b.ld(rx, ox, L.oMxh);
    m.xe = b.ld(rx, ox, L.oMxe);
    return m;
}

__device__ __forceinline__ void bandk_mem_store(const RBuf& b, const StateLayout& L, const Geo& g, int y, int x,
                                                bool own, const CellMem& m)
{
    const bool ry = own && flag_hy(g, y), rx = own && flag_hx(g, x);
    const uint32_t oy = (uint32_t)((ry ? band_y(g, y) : 0) * g.nx + x) * 4u;
    const uint32_t ox = (uint32_t)(y * g.bx + (rx ? band_x(g, x) : 0)) * 4u;
    b.st(ry, m.yh, oy, L.oMyh);
    b.st(ry, m.ye, oy, L.oMye);
    b.st(rx, m.xh, ox, L.oMxh);
    b.st(rx, m.xe, ox, L.oMxe);
}

// A filter on a register memory: the recursion where the site applies,
// the identity elsewhere.  The coefficients are read whether or not the
// site applies (every row and column has table entries), so the reads
// leave with the stencil's instead of after it: one LDS round trip less
// per filtered update.
__device__ __forceinline__ float rsite(bool on, float& m, const float* tab, int n, float d)
{
    const float a = tab[0], b = tab[n], ik = tab[2 * n];
    float mn = m;
    const float r = cpml_step(mn, a, b, ik, d);
    m = on ? mn : m;
    return on ? r : d;
}

// Exchange number n, in two halves that need no barrier of their own.
// Publish: the words of the cells on the first and last hd own rows (w[0..6]
// of each cell, read by get(i, k); each thread publishes its own cells,
// whose values it wrote itself).
template <int P, int CK, typename Get>
__device__ __forceinline__ void bandk_publish(const BandKArgs& ba, const BandK& t, const int (&pk)[CK], int n,
                                              Get get)
{
    const int nx = ba.a.g.nx, hd = ba.hd;
    const size_t plane = (size_t)hd * nx, side_w = plane * BK_NW;   // one word of every cell of a side
    const uint64_t tag = (uint64_t)(uint32_t)(n + 1) << 32;
    uint64_t* ob = ba.xbuf + (size_t)((t.w * 2 + (n & 1)) * 2) * side_w;
#pragma unroll
    for (int i = 0; i < CK; ++i) {
        const Cell c = cell(pk[i]);
        const int y = c.y(), x = c.j() - (y - t.y_arr) * nx;
        const bool valid = c.j() < (t.eb - t.y_arr) * nx && y >= t.ya && y < t.yb;
        if (!valid) continue;
        if (y < t.ya + hd) {                                  // side 0: first hd own rows
            uint64_t* o = ob + (size_t)(y - t.ya) * nx + x;
#pragma unroll
            for (int k = 0; k < BK_NW; ++k)
                __hip_atomic_store(&o[k * plane], tag | __float_as_uint(get(i, k)), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        if (y >= t.yb - hd) {                                 // side 1: last hd own rows
            uint64_t* o = ob + side_w + (size_t)(y - (t.yb - hd)) * nx + x;
#pragma unroll
            for (int k = 0; k < BK_NW; ++k)
                __hip_atomic_store(&o[k * plane], tag | __float_as_uint(get(i, k)), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Poll: wait for the neighbours' words of exchange n for the cells on the
// extended rows outside the band and hand them to put(i, k, v).  Returns
// false when this thread's wait failed or the launch has failed (err is
// then set); the caller tells the other threads at its next barrier.
//
// The words go through the memory that all the chip's L2s share, so each
// poll is one memory round trip; neighbours publish at about the same time,
// and a poll sent at once mostly arrives before their words and costs a
// second round trip.  A thread with cells to poll therefore sleeps
// BK_POLL_WAIT units (64 clocks each) before its first poll: on the 86^2
// order-2 grid (300 steps, an exchange every third) 20 units give the
// forward 360 us and the adjoint 419 us, against 380 / 437 us at 10 units,
// 364 / 424 at 15 and 362 / 421 at 25.
constexpr int BK_POLL_WAIT = 20;

template <int P, int CK, typename Put>
__device__ __forceinline__ bool bandk_poll(const BandKArgs& ba, const BandK& t, const int (&pk)[CK], int n, Put put)
{
    const int nx = ba.a.g.nx, hd = ba.hd;
    const size_t plane = (size_t)hd * nx, side_w = plane * BK_NW;
    const uint64_t tag = (uint64_t)(uint32_t)(n + 1) << 32;
    bool bad = ba.spin_max <= 0;                              // (a host-forced failure, for tests)
    bool waited = false;
#pragma unroll
    for (int i = 0; i < CK; ++i) {
        const Cell c = cell(pk[i]);
        const int y = c.y(), x = c.j() - (y - t.y_arr) * nx;
        const bool valid = c.j() < (t.eb - t.y_arr) * nx;
        if (!valid || bad || (y >= t.ya && y < t.yb)) continue;
        // above the band: the band above's last rows [ya - hd, ya); below:
        // the band below's first rows [yb, yb + hd)
        const bool above = y < t.ya;
        const int nb = above ? t.b - 1 : t.b + 1;
        const int r = above ? y - (t.ya - hd) : y - t.yb;
        const uint64_t* ib = ba.xbuf + (size_t)(((t.s * ba.nband + nb) * 2 + (n & 1)) * 2 + (above ? 1 : 0)) * side_w +
                             (size_t)r * nx + x;
        uint64_t w[BK_NW];
        if (!waited) __builtin_amdgcn_s_sleep(BK_POLL_WAIT);
        waited = true;
        for (int it = 0;; ++it) {
            bool all = true;
#pragma unroll
            for (int k = 0; k < BK_NW; ++k) {
                w[k] = __hip_atomic_load(&ib[k * plane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                all = all && (w[k] & 0xffffffff00000000ull) == tag;
            }
            if (all) break;
            if (it >= ba.spin_max ||
                ((it & 63) == 63 && __hip_atomic_load(ba.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))) {
                bad = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (bad) continue;
#pragma unroll
        for (int k = 0; k < BK_NW; ++k) put(i, k, __uint_as_float((uint32_t)w[k]));
    }
    if (bad) __hip_atomic_store(ba.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return !bad;
}

// Forward, blocked: steps t0 .. t1-1, workgroup = (shot, band).
template <int P, int SNAP, int CK>
__global__ __launch_bounds__(NTS) void k_fwd_bandk(BandKArgs ba)
{
    extern __shared__ float lds[];
    __shared__ int quit;
    const SmallArgs& a = ba.a;
    const Geo& g = a.g;
    const StateLayout& L = a.L;
    const BandK t = bandk_of(ba);
    const int s = t.s, tid = threadIdx.x;
    const int nth = CK == 1 ? (int)blockDim.x : NTS;   // threads (bandk_threads)
    const int ny = g.ny, nx = g.nx;
    const int rows = ba.rb + 2 * ba.hd;
    const BandKLayout bl = bandk_layout(g, ba.rb, ba.hd, 3);
    float* const sE = lds + bl.pad;
    float* const sHx = sE + bl.stride;
    float* const sHz = sHx + bl.stride;
    const float* const ty = lds + bl.ty;
    const float* const tx = lds + bl.tx;
    const int* const slot = reinterpret_cast<const int*>(lds + bl.slot);

    const RBuf b0(a.set0 + (int64_t)s * L.shot_bytes, L.shot_bytes);
    const RBuf b1(a.set1 + (int64_t)s * L.shot_bytes, L.shot_bytes);
    const RBuf bm(a.m.base + (int64_t)s * a.m.shot_stride, a.m.bytes);
    const RBuf bev(a.ev.base, a.ev.bytes);

    // fields of the array rows (0 off the grid) and the padding
    const int arr = rows * nx;
    for (int i = tid - (int)bl.pad; i < arr + (int)bl.pad; i += nth) {
        const int gj = t.y_arr * nx + i;
        const bool in = i >= 0 && i < arr && gj >= 0 && gj < ny * nx;
        const uint32_t o = (uint32_t)(in ? gj : 0) * 4u;
        sE[i] = b0.ld(in, o, L.oE);
        sHx[i] = b0.ld(in, o, L.oHx);
        sHz[i] = b0.ld(in, o, L.oHz);
    }
    bandk_tables(lds, bl, g, a.cp, a.ev, s, nth);
    if (tid == 0) quit = 0;

    auto xof = [&](const Cell& c) { return c.j() - (c.y() - t.y_arr) * nx; };
    // iteration i of the cell loops has work in this wave
    const BandKCells cs = bandk_cells(t, g);
    const int wbase = __builtin_amdgcn_readfirstlane(tid & ~63), ncel = cs.n;
    auto live = [&](int i) { return i * nth + wbase < ncel; };
    int pk[CK];
    float ca[CK], cb[CK], cq[CK];
    CellMem mm[CK];
#pragma unroll
    for (int i = 0; i < CK; ++i) {
        const int je = tid + i * nth;
        const bool ok = je < cs.n;
        pk[i] = pack_bandk_cell<P>(je, t, cs, rows, g);
        const Cell c0{pk[i]};
        const uint32_t o = (uint32_t)(ok ? c0.y() * nx + xof(c0) : 0) * 4u;
        ca[i] = bm.ld(ok, o, a.m.oCa);
        cb[i] = bm.ld(ok, o, a.m.oCb);
        cq[i] = bm.ld(ok, o, a.m.oCq);
        const Cell c{pk[i]};
        mm[i] = bandk_mem_load(b0, L, g, c.y(), xof(c), ok);
    }
    __syncthreads();

    // event-row offsets of the cells (RBuf::OOB off the event rows), and
    // the iterations in which this wave has any
    int evo[CK], evmask = 0;
#pragma unroll
    for (int i = 0; i < CK; ++i) {
        const Cell c{pk[i]};
        const int gs = slot[c.y()];
        evo[i] = c.bit(CB_E) && gs >= 0 ? (gs * nx + xof(c)) * 4 : RBuf::OOB;
        if (__builtin_amdgcn_ballot_w64(evo[i] != RBuf::OOB) != 0) evmask |= 1 << i;
    }
    evmask = __builtin_amdgcn_readfirstlane(evmask);

    // source amplitudes of the cells on event rows: two steps ahead, in two
    // sets (steps of even and odd offset from t0), each reloaded right
    // after its step has used it
    auto load_add = [&](int tt, float (&dst)[CK]) {
        const bool in_run = tt < a.t1;
        const uint32_t off = a.ev_add0 + (uint32_t)(in_run ? tt - a.t0 : 0) * a.ev_row;
#pragma unroll
        for (int i = 0; i < CK; ++i) {
            dst[i] = 0.0f;
            if (((evmask >> i) & 1) == 0) continue;
            dst[i] = bev.ldv(in_run ? evo[i] : RBuf::OOB, off);
        }
    };
    float add0[CK], add1[CK];
    load_add(a.t0, add0);
    load_add(a.t0 + 1, add1);
    auto get = [&](int i, int k) -> float {
        const int j = Cell{pk[i]}.j();
        return k == 0 ? sE[j] : k == 1 ? sHx[j] : k == 2 ? sHz[j] : k == 3 ? mm[i].yh : k == 4 ? mm[i].xh
             : k == 5 ? mm[i].ye : mm[i].xe;
    };
    auto put = [&](int i, int k, float v) {
        const int j = Cell{pk[i]}.j();
        if (k == 0) sE[j] = v;
        else if (k == 1) sHx[j] = v;
        else if (k == 2) sHz[j] = v;
        else if (k == 3) mm[i].yh = v;
        else if (k == 4) mm[i].xh = v;
        else if (k == 5) mm[i].ye = v;
        else mm[i].xe = v;
    };

    int nex = 0, xc = 0;                    // exchanges done, steps since the last one
    StepPhase sp;                           // of the step
    if constexpr (SNAP != SNAP_NONE) sp.init(a.t0, a.R);
    // one step; false when the launch has failed
    auto step = [&](int tt, float (&add)[CK]) -> bool {
        // ---- H half-step on every extended row
#pragma unroll
        for (int i = 0; i < CK; ++i) {
            if (!live(i)) continue;
            const Cell c = bcell<P>(pk[i]);
            const int j = c.j(), x = xof(c);
            const float hx = sHx[j], hz = sHz[j];
            float dy = g.rdy * stencil<P>([&](int k) { return sE[j + k * nx]; },
                                          [&](int k) { return sE[j - (k - 1) * nx]; });
            float dx = g.rdx * stencil<P>([&](int k) { return sE[j + k]; }, [&](int k) { return sE[j - k + 1]; });
            dy = rsite(c.bit(CB_FHY), mm[i].yh, ty + c.y(), ny, dy);
            dx = rsite(c.bit(CB_FHX), mm[i].xh, tx + x, nx, dx);
            sHx[j] = c.bit(CB_HX) ? fmaf(-cq[i], dy, hx) : hx;
            sHz[j] = c.bit(CB_HZ) ? fmaf(cq[i], dx, hz) : hz;
        }
        __syncthreads();

        // ---- E step on every extended row; outputs of the own rows
        const bool stored = SNAP != SNAP_NONE && sp.ph == 0;
        const RBuf bsp(stored ? a.snap + (uint64_t)sp.idx * a.snap_stride + (uint64_t)s * a.snap_shot_bytes
                              : nullptr,
                       stored ? a.snap_shot_bytes : 0u);
        if constexpr (SNAP != SNAP_NONE) sp.next(a.R);
        const uint32_t out_off = a.ev_out0 + (uint32_t)(tt - a.t0) * a.ev_row;
        const bool next_in = tt + 2 < a.t1;
        const uint32_t next_off = a.ev_add0 + (uint32_t)(next_in ? tt + 2 - a.t0 : 0) * a.ev_row;
#pragma unroll
        for (int i = 0; i < CK; ++i) {
            if (!live(i)) continue;
            const Cell c = bcell<P>(pk[i]);
            const int j = c.j(), y = c.y(), x = xof(c);
            const float ev = sE[j];
            float uu = g.rdx * stencil<P>([&](int k) { return sHz[j + k - 1]; }, [&](int k) { return sHz[j - k]; });
            float v = g.rdy * stencil<P>([&](int k) { return sHx[j + (k - 1) * nx]; },
                                         [&](int k) { return sHx[j - k * nx]; });
            uu = rsite(c.bit(CB_FEX), mm[i].xe, tx + 3 * nx + x, nx, uu);
            v = rsite(c.bit(CB_FEY), mm[i].ye, ty + 3 * ny + y, ny, v);
            const float curl = uu - v;
            const bool own = y >= t.ya && y < t.yb;
            if constexpr (SNAP != SNAP_NONE) {
                const bool in_w = own && c.bit(CB_E) && y >= g.y0 && y < g.y1 && x >= g.x0 && x < g.x1;
                snap_put2<SNAP>(bsp, stored && in_w, (uint32_t)((y - g.y0) * g.nxi + (x - g.x0)), ev, curl);
            }
            float en = fmaf(ca[i], ev, cb[i] * curl);
            en = evo[i] != RBuf::OOB ? en + add[i] : en;
            if ((evmask >> i) & 1) {
                bev.stv(en, own ? evo[i] : RBuf::OOB, out_off);
                add[i] = bev.ldv(next_in ? evo[i] : RBuf::OOB, next_off);   // step tt + 2
            }
            sE[j] = c.bit(CB_E) ? en : ev;
        }
        if (++xc == ba.kx) xc = 0;
        if (tt + 1 < a.t1 && xc == 0) {
            // Own cells' values are final (each thread wrote its own), so
            // publish and poll at once.  The neighbours' fields go straight
            // into the outer rows while other threads may still run this
            // step's E update: of the rows written, that update reads only
            // Hx on the P rows next to the band (for own cells), whose values
            // here are already exact, so the stores do not change them; the
            // other reads are for outer-row cells, whose results the
            // exchange replaces.  The next reads follow the barrier below.
            bandk_publish<P, CK>(ba, t, pk, nex, get);
            if (!bandk_poll<P, CK>(ba, t, pk, nex, put)) quit = 1;
            ++nex;
        }
        __syncthreads();
        return quit == 0;
    };
    drain_vmem();
    for (int tt = a.t0; tt < a.t1; tt += 2) {
        if (!step(tt, add0)) break;
        if (tt + 1 < a.t1 && !step(tt + 1, add1)) break;
    }

    // own rows back
#pragma unroll
    for (int i = 0; i < CK; ++i) {
        const Cell c{pk[i]};
        const int y = c.y(), x = xof(c);
        const bool own = c.j() < (t.eb - t.y_arr) * nx && y >= t.ya && y < t.yb;
        const uint32_t o = (uint32_t)(own ? y * nx + x : 0) * 4u;
        b1.st(own, sE[c.j()], o, L.oE);
        b1.st(own, sHx[c.j()], o, L.oHx);
        b1.st(own, sHz[c.j()], o, L.oHz);
        bandk_mem_store(b1, L, g, y, x, own, mm[i]);
    }
}

// Exact adjoint, blocked: steps t1-1 down to t0, workgroup = (shot, band).
template <int P, int SNAP, int CK>
__global__ __launch_bounds__(NTS) void k_adj_bandk(BandKArgs ba)
{
    extern __shared__ float lds[];
    __shared__ int quit;
    const SmallArgs& a = ba.a;
    const Geo& g = a.g;
    const StateLayout& L = a.L;
    const BandK t = bandk_of(ba);
    const int s = t.s, tid = threadIdx.x;
    const int nth = CK == 1 ? (int)blockDim.x : NTS;   // threads (bandk_threads)
    const int ny = g.ny, nx = g.nx;
    const int rows = ba.rb + 2 * ba.hd;
    const BandKLayout bl = bandk_layout(g, ba.rb, ba.hd, 4);
    float* const sU = lds + bl.pad;
    float* const sW = sU + bl.stride;
    float* const sTZ = sW + bl.stride;
    float* const sTX = sTZ + bl.stride;
    const float* const ty = lds + bl.ty;
    const float* const tx = lds + bl.tx;
    const int* const slot = reinterpret_cast<const int*>(lds + bl.slot);

    const RBuf b0(a.set0 + (int64_t)s * L.shot_bytes, L.shot_bytes);
    const RBuf b1(a.set1 + (int64_t)s * L.shot_bytes, L.shot_bytes);
    const RBuf bm(a.m.base + (int64_t)s * a.m.shot_stride, a.m.bytes);
    const RBuf bev(a.ev.base, a.ev.bytes);
    const uint32_t slab_b = (uint32_t)(g.slab * 4);
    const RBuf bga(a.gca + (int64_t)s * g.slab, a.gca ? slab_b : 0u);
    const RBuf bgb(a.gcb + (int64_t)s * g.slab, a.gcb ? slab_b : 0u);

    for (int i = tid; i < 4 * (int)bl.stride; i += nth) lds[i] = 0.0f;
    bandk_tables(lds, bl, g, a.cp, a.ev, s, nth);
    if (tid == 0) quit = 0;

    auto xof = [&](const Cell& c) { return c.j() - (c.y() - t.y_arr) * nx; };
    auto own_of = [&](const Cell& c) {
        const int y = c.y();
        return c.j() < (t.eb - t.y_arr) * nx && y >= t.ya && y < t.yb;
    };
    auto in_window = [&](const Cell& c) {
        const int y = c.y(), x = xof(c);
        return own_of(c) && c.bit(CB_E) && y >= g.y0 && y < g.y1 && x >= g.x0 && x < g.x1;
    };
    const BandKCells cs = bandk_cells(t, g);
    const int wbase = __builtin_amdgcn_readfirstlane(tid & ~63), ncel = cs.n;
    auto live = [&](int i) { return i * nth + wbase < ncel; };
    int pk[CK];
    float ca[CK], cb[CK], cq[CK], lE[CK], lHx[CK], lHz[CK], ga[CK], gb[CK];
    CellMem mm[CK];
#pragma unroll
    for (int i = 0; i < CK; ++i) {
        const int je = tid + i * nth;
        const bool ok = je < cs.n;
        pk[i] = pack_bandk_cell<P>(je, t, cs, rows, g);
        const Cell c0{pk[i]};
        const uint32_t o = (uint32_t)(ok ? c0.y() * nx + xof(c0) : 0) * 4u;
        ca[i] = bm.ld(ok, o, a.m.oCa);
        cb[i] = bm.ld(ok, o, a.m.oCb);
        cq[i] = bm.ld(ok, o, a.m.oCq);
        lE[i] = b0.ld(ok, o, L.oE);
        lHx[i] = b0.ld(ok, o, L.oHx);
        lHz[i] = b0.ld(ok, o, L.oHz);
        const Cell c{pk[i]};
        const bool gw = SNAP != SNAP_NONE && in_window(c);
        ga[i] = bga.ld(gw, o, 0u);
        gb[i] = bgb.ld(gw, o, 0u);
        mm[i] = bandk_mem_load(b0, L, g, c.y(), xof(c), ok);
    }

    int evo[CK];   // event-row offsets of the cells, set once the tables are in LDS
    // residuals at the receivers and snapshots of a step: two steps ahead,
    // in two sets (steps of even and odd offset from t1 - 1), each reloaded
    // right after its step's phase 1 has used it
    StepPhase lp;                           // of the step load_step reads (one lower at each call)
    if constexpr (SNAP != SNAP_NONE) lp.init(a.t1 - 1, a.R);
    auto load_step = [&](int tt, float (&add)[CK], float (&se)[CK], float (&sc)[CK]) {
        const bool in_run = tt >= a.t0;
        const uint32_t off = a.ev_add0 + (uint32_t)(in_run ? tt - a.t0 : 0) * a.ev_row;
        const bool stored = SNAP != SNAP_NONE && in_run && lp.ph == 0;
        const RBuf bsp(stored ? a.snap + (uint64_t)lp.idx * a.snap_stride + (uint64_t)s * a.snap_shot_bytes
                              : nullptr,
                       stored ? a.snap_shot_bytes : 0u);
        if constexpr (SNAP != SNAP_NONE) lp.prev(a.R);
        // (every wave loads, off the buffers where it has no cell, so that
        // the registers are only ever written by loads: no wait for the
        // previous loads into them)
#pragma unroll
        for (int i = 0; i < CK; ++i) {
            const Cell c = bcell<P>(pk[i]);
            const int y = c.y(), x = xof(c);
            add[i] = bev.ldv(in_run ? evo[i] : RBuf::OOB, off);
            const SnapPair sp = snap_get2<SNAP>(bsp, stored && in_window(c),
                                                (uint32_t)((y - g.y0) * g.nxi + (x - g.x0)));
            se[i] = sp.e;
            sc[i] = sp.c;
        }
    };
    auto get = [&](int i, int k) -> float {
        return k == 0 ? lE[i] : k == 1 ? lHx[i] : k == 2 ? lHz[i] : k == 3 ? mm[i].yh : k == 4 ? mm[i].xh
             : k == 5 ? mm[i].ye : mm[i].xe;
    };
    auto put = [&](int i, int k, float v) {
        if (k == 0) lE[i] = v;
        else if (k == 1) lHx[i] = v;
        else if (k == 2) lHz[i] = v;
        else if (k == 3) mm[i].yh = v;
        else if (k == 4) mm[i].xh = v;
        else if (k == 5) mm[i].ye = v;
        else mm[i].xe = v;
    };
    __syncthreads();
    // event-row offsets of the cells (RBuf::OOB off the event rows)
#pragma unroll
    for (int i = 0; i < CK; ++i) {
        const Cell c{pk[i]};
        const int gs = slot[c.y()];
        evo[i] = c.bit(CB_E) && gs >= 0 ? (gs * nx + xof(c)) * 4 : RBuf::OOB;
    }
    float add0[CK], se0[CK], sc0[CK], add1[CK], se1[CK], sc1[CK];
    load_step(a.t1 - 1, add0, se0, sc0);
    load_step(a.t1 - 2, add1, se1, sc1);

    int nex = 0, xc = 0;                    // exchanges done, steps since the last one
    StepPhase sp;                           // of the step
    if constexpr (SNAP != SNAP_NONE) sp.init(a.t1 - 1, a.R);
    // one step; false when the launch has failed
    auto step = [&](int tt, float (&add)[CK], float (&se)[CK], float (&sc)[CK]) -> bool {
        const bool stored = SNAP != SNAP_NONE && sp.ph == 0;
        if constexpr (SNAP != SNAP_NONE) sp.prev(a.R);
        const uint32_t out_off = a.ev_out0 + (uint32_t)(tt - a.t0) * a.ev_row;

        // ---- phase 1 on every extended row: residual, gradient (own), Cb, E-update filters
#pragma unroll
        for (int i = 0; i < CK; ++i) {
            if (!live(i)) continue;
            const Cell c = bcell<P>(pk[i]);
            const int j = c.j(), y = c.y(), x = xof(c);
            const bool on = c.bit(CB_E);
            const float e = evo[i] != RBuf::OOB ? lE[i] + add[i] : lE[i];
            bev.stv(e, own_of(c) ? evo[i] : RBuf::OOB, out_off);
            if (SNAP != SNAP_NONE && stored) {
                const bool in_w = in_window(c);
                const float na = fmaf(e, se[i] * a.ratio, ga[i]), nb = fmaf(e, sc[i] * a.ratio, gb[i]);
                ga[i] = in_w ? na : ga[i];
                gb[i] = in_w ? nb : gb[i];
            }
            const float hv = cb[i] * e;
            const float u = rsite(c.bit(CB_FEX), mm[i].xe, tx + 3 * nx + x, nx, hv);
            const float w = rsite(c.bit(CB_FEY), mm[i].ye, ty + 3 * ny + y, ny, hv);
            sU[j] = on ? u : 0.0f;
            sW[j] = on ? w : 0.0f;
            lE[i] = e;
        }
        load_step(tt - 2, add, se, sc);
        __syncthreads();
        if (quit) return false;                 // an exchange wait failed (set before this barrier)

        // ---- phase 2 on every extended row: transposed curl, Cq, H-update filters
#pragma unroll
        for (int i = 0; i < CK; ++i) {
            if (!live(i)) continue;
            const Cell c = bcell<P>(pk[i]);
            const int j = c.j();
            const float accx = stencil<P>([&](int k) { return sW[j + k * nx]; },
                                          [&](int k) { return sW[j - (k - 1) * nx]; });
            const float accz = stencil<P>([&](int k) { return sU[j + k]; }, [&](int k) { return sU[j - k + 1]; });
            const float lhx = fmaf(g.rdy, accx, lHx[i]);
            const float lhz = fmaf(-g.rdx, accz, lHz[i]);
            const int y = c.y(), x = xof(c);
            const float txv = rsite(c.bit(CB_FHY), mm[i].yh, ty + y, ny, cq[i] * lhx);
            const float tz = rsite(c.bit(CB_FHX), mm[i].xh, tx + x, nx, cq[i] * lhz);
            const bool hx = c.bit(CB_HX), hz = c.bit(CB_HZ);
            lHx[i] = hx ? lhx : lHx[i];
            lHz[i] = hz ? lhz : lHz[i];
            sTX[j] = hx ? txv : 0.0f;
            sTZ[j] = hz ? tz : 0.0f;
        }
        __syncthreads();

        // ---- phase 3 on every extended row: lambda_E = Ca e - Dx[t_z] + Dz[t_x]
#pragma unroll
        for (int i = 0; i < CK; ++i) {
            if (!live(i)) continue;
            const Cell c = bcell<P>(pk[i]);
            const int j = c.j();
            const float az = stencil<P>([&](int k) { return sTZ[j + k - 1]; }, [&](int k) { return sTZ[j - k]; });
            const float ay = stencil<P>([&](int k) { return sTX[j + (k - 1) * nx]; },
                                        [&](int k) { return sTX[j - k * nx]; });
            const float en = fmaf(ca[i], lE[i], fmaf(-az, g.rdx, ay * g.rdy));
            lE[i] = c.bit(CB_E) ? en : lE[i];
        }
        if (++xc == ba.kx) xc = 0;
        if (tt > a.t0 && xc == 0) {
            // the state lives in the cells' registers: no barrier (the next
            // one, after phase 1, reports a failed wait to every thread)
            bandk_publish<P, CK>(ba, t, pk, nex, get);
            if (!bandk_poll<P, CK>(ba, t, pk, nex, put)) quit = 1;
            ++nex;
        }
        return true;
    };
    drain_vmem();
    for (int tt = a.t1 - 1; tt >= a.t0; tt -= 2) {
        if (!step(tt, add0, se0, sc0)) break;
        if (tt - 1 >= a.t0 && !step(tt - 1, add1, se1, sc1)) break;
    }

#pragma unroll
    for (int i = 0; i < CK; ++i) {
        const Cell c{pk[i]};
        const int y = c.y(), x = xof(c);
        const bool own = own_of(c);
        const uint32_t o = (uint32_t)(own ? y * nx + x : 0) * 4u;
        b1.st(own, lE[i], o, L.oE);
        b1.st(own, lHx[i], o, L.oHx);
        b1.st(own, lHz[i], o, L.oHz);
        const bool gw = SNAP != SNAP_NONE && in_window(c);
        bga.st(gw, ga[i], o, 0u);
        bgb.st(gw, gb[i], o, 0u);
        bandk_mem_store(b1, L, g, y, x, own, mm[i]);
    }
}

}  // namespace tmf
