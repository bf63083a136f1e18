// Two forward time steps per launch (temporal blocking), gfx950 / wave64.
//
// k_fwd_step2 advances every shot from step n to step n+2 in one pass over
// the state: stage A computes the step n -> n+1 exactly as k_fwd_step does,
// and stage B consumes stage A's rows while they are still in registers and
// LDS and computes the step n+1 -> n+2.  The state crosses HBM once per two
// steps; the intermediate state never leaves the chip.
//
// Streaming (iteration r, one row per stage):
//   stage A: H row hA = r - P,    E row yA = r - 2P + 1   (as k_fwd_step)
//   stage B: H row hB = r - 3P+1, E row yB = r - 4P + 2
// Stage B needs the E^{n+1} rows up to yA (register window ewB), the old
// H^{n+1/2} of row hB (the oldest Hx row of stage A's window; Hz from a ring
// of 2P rows in LDS) and the CPML memories stage A produced for its rows,
// which wait 2P-1 iterations in a lane-private LDS FIFO (each lane reads
// back only what it wrote, so the FIFO needs no barrier).  The model
// coefficients of stage B's rows are loaded again (they were read 2P-1 rows
// earlier by the same workgroup and are served by the caches).
//
// A strip of 256 lanes owns up to W = 256 - 8P + 4 columns (the strips of
// a grid are cut to equal widths, Tiling::W): stage A's values are
// valid 2P-1 lanes further in from the edges than the loaded E^n, stage B's
// another 2P-1.  A chunk of CH owned rows reads 4P-2 rows above and below.
// Values of stage A outside the field's index set are forced to 0 exactly
// as the untouched cells of the single-step path stay 0, and every
// operation is written as in k_fwd_step, so both kernels give bitwise the
// same state.
//
// Sources and receivers of both steps are handled inside the kernel through
// the event rows (EventRows): the add row of step n is added to E^{n+1} at
// every lane that computes the row, halo lanes included, and the owner
// keeps the result; stage B does the same for step n+1 on its owned output
// rows.
//
// Fast blocks: most unrolled blocks of a chunk lie where every stage is
// active, no row is a CPML band row or carries sources or receivers, and
// every row is owned or inside the index sets.  Those blocks run an
// instance of the iteration with all row predicates folded away: loads and
// stores use a loop-invariant lane offset (out of range where the lane is
// masked) plus a uniform row offset, so they cost no vector instructions
// for addressing.  The other blocks run the general iteration.  Both compute
// the same values.
#pragma once

#include <type_traits>

#include "tm_step.hpp"

namespace tmf {

constexpr int CH2_MAX = 128;   // largest chunk height of the two-step kernel (LDS tables)
constexpr int PREFETCH_F2 = 1; // rows of loads in flight ahead
constexpr int UNROLL_F2 = 4;   // row-loop unroll, a multiple of PREFETCH_F2
constexpr int UNROLL_F2_CX = 2; // ... of the compact-FIFO instances (order 8, four workgroups per CU)
constexpr int XFIFO_W = 56;     // x-band lanes per strip the compact FIFOs hold

template <int P>
struct Strip2 {
    static constexpr int W = NT - 8 * P + 4;   // most owned columns per strip
    static constexpr int OFF = 4 * P - 2;      // lane of the first owned column
};

struct Fwd2Args {
    Geo g;
    Tiling t;
    StateLayout L;
    Model m;
    const float* __restrict__ cp;      // CPML table [12][L]
    const char* __restrict__ set0;     // state at step n
    char* __restrict__ set1;           // state at step n+2
    char* __restrict__ snap0;          // (Ey^n, curl H^n) pairs [S][nyi][nxi][2], or null (step n not stored)
    char* __restrict__ snap1;          // (Ey^{n+1}, curl H^{n+1}) pairs, or null
    uint32_t snap_shot_bytes;          // bytes of one shot's pairs
    EventRows ev;                      // sources (add) and receivers (out)
    EventStep es0, es1;                // ... of steps n and n+1
    float cq;                          // Cq where it holds one value (UQ instances)
};

// UQ: Cq holds one value in every cell (mu_r uniform, non-magnetic media),
// so no Cq bytes are read: each Cq load becomes that value on the lanes and
// rows where the load would have read a cell and 0 elsewhere, and the step
// computes bitwise what it computes with the array.
// CX (order 8): the FIFOs of stage A's x-band memories hold only the
// strip's x-band lanes (at most XFIFO_W, which the plan checks); the other
// lanes' memory is 0, which is what they hold in the full FIFOs (their
// CPML coefficients are a = b = 0).  With an unroll of two this fits the
// kernel into 128 VGPRs and 40 KB of LDS, four workgroups per CU.
template <int P, int SNAP, bool UQ, bool CX>
__global__ __launch_bounds__(NT, (CX || P <= 2) ? 4 : 3) void k_fwd_step2(Fwd2Args a)
{
    constexpr int OFF = Strip2<P>::OFF;
    constexpr int D = PREFETCH_F2;
    constexpr int U = CX ? UNROLL_F2_CX : UNROLL_F2;
    constexpr int XW = XFIFO_W;                     // x-band slots of the compact FIFOs
    constexpr int R2 = 2 * P;                       // ring / FIFO depth (a power of two)
    constexpr uint32_t ESZ = snap_bytes<SNAP>();
    __shared__ float rowA[2][NT];                   // E^n row hA, by row parity
    __shared__ float rowB[2][NT];                   // E^{n+1} row hB, by row parity
    __shared__ float ringA[R2][NT];                 // Hz^{n+1/2} rows
    __shared__ float ringB[P][NT];                  // Hz^{n+3/2} rows
    // stage A's CPML memories for stage B, each [R2] rows: full layout
    // [Myh | Mxh | Mxe | Mye] of NT lanes; CX: [Myh | Mye] of NT lanes, then
    // [Mxh | Mxe] of XW x-band slots
    __shared__ float fifo[CX ? 2 * R2 * (NT + XW) : 4 * R2 * NT];
    __shared__ float cyt[CH2_MAX + 6 * P - 3][6];   // per-row CPML coefficients
    __shared__ int evs[CH2_MAX + 4 * P - 2];        // slot of each stage-A E row
    __shared__ int ev_lo, ev_hi;                    // first / last stage-A E row with events

    const Geo& g = a.g;
    const StateLayout& L = a.L;
    int s, strip, ya, yb;
    tile2_of(a.t, g.ny, P, s, strip, ya, yb);
    const int tid = threadIdx.x;
    const int nx = g.nx, ny = g.ny;
    const int xs = P + strip * a.t.W;               // a.t.W <= Strip2<P>::W
    const int xe = min(xs + a.t.W, nx - P + 1);
    const int yc0 = ya - 3 * P + 1;                 // first row of the CPML table
    const int ye0 = ya - 2 * P + 1;                 // first stage-A E row
    if (tid == 0) {
        ev_lo = INT32_MAX;
        ev_hi = INT32_MIN;
    }
    __syncthreads();
    load_row_cpml(cyt, a.cp, g, yc0, yb - ya + 6 * P - 3);
    load_row_slots(evs, &ev_lo, &ev_hi, a.ev.row_slot, s, ny, ye0, yb - ya + 4 * P - 2);
    __syncthreads();

    const int c = xs - OFF + tid;                   // this lane's column
    const bool own = (c >= xs) & (c < xe);
    const bool incol = (c >= 0) & (c < nx);
    const bool colE = (c >= P) & (c <= nx - P);     // Ey and Hx columns
    const bool colHz = (c >= P) & (c <= nx - P - 1);
    // lanes whose stencil inputs are all valid, per stage
    const bool hzA_ok = colHz & (tid >= P - 1) & (tid <= NT - P - 1);
    const bool eA_ok = colE & (tid >= 2 * P - 1) & (tid <= NT - 2 * P);
    const bool hzB_ok = colHz & (tid >= 3 * P - 2) & (tid <= NT - 3 * P);
    const bool fx_h = incol & ((c < g.x0) | (c >= g.hx1));
    const bool fx_e = incol & ((c < g.x0) | (c >= g.x1));
    const bool in_x = (c >= g.x0) & (c < g.x1);
    const int c0 = xs - OFF;
    const bool xband = c0 < g.x0 || c0 + NT - 1 >= g.hx1;   // uniform
    // x-band FIFO slot: the lane itself, or (CX) the lane's index among the
    // strip's x-band lanes, -1 off the band
    int xi = tid;
    if constexpr (CX) {
        const int cl = max(c0, 0), cr = max(g.hx1, c0);
        const int nl = max(0, min(g.x0, c0 + NT) - cl);
        xi = !fx_h ? -1 : (c < g.x0 ? c - cl : nl + (c - cr));
    }
    // k = 0: the H-update memory, 1: the E-update memory
    auto yref = [&](int k, int slot) -> float& {
        return fifo[((CX ? k : 3 * k) * R2 + slot) * NT + tid];
    };
    auto xput = [&](int k, int slot, float m) {
        if constexpr (CX) {
            if (xi >= 0) fifo[2 * R2 * NT + (k * R2 + slot) * XW + xi] = m;
        } else {
            fifo[((1 + k) * R2 + slot) * NT + tid] = m;
        }
    };
    auto xget = [&](int k, int slot) {
        if constexpr (CX) {
            const float m = fifo[2 * R2 * NT + (k * R2 + slot) * XW + max(xi, 0)];
            return xi < 0 ? 0.0f : m;
        } else {
            return fifo[((1 + k) * R2 + slot) * NT + tid];
        }
    };
    const int bxc = band_x(g, incol ? c : 0);
    const int th = min(max(tid, P - 1), NT - P - 1);
    const int te = min(max(tid, P), NT - P);

    Cpml1 cx_h{0.f, 0.f, 1.f}, cx_e{0.f, 0.f, 1.f};
    if (fx_h) cx_h = cpml_at(a.cp, g.L, AXH, c);
    if (fx_e) cx_e = cpml_at(a.cp, g.L, AX, c);

    auto in_rows = [&](int y) { return (y >= 0) & (y < ny); };
    auto rowE = [&](int y) { return (y >= P) & (y <= ny - P); };
    auto hx_row = [&](int h) { return (h >= P) & (h <= ny - P - 1); };
    auto hz_row = [&](int h) { return (h >= P) & (h <= ny - P); };
    auto own_row = [&](int y) { return (y >= ya) & (y < yb); };
    auto fy_h = [&](int h) { return (h < g.y0) | (h >= g.hy1); };
    auto fy_e = [&](int y) { return (y < g.y0) | (y >= g.y1); };
    auto slot2 = [&](int y) { return (y + 4 * P) & (R2 - 1); };   // y >= -4P
    auto slot1 = [&](int y) { return (y + 4 * P) & (P - 1); };

    const RBuf b0(a.set0 + (int64_t)s * L.shot_bytes, L.shot_bytes);
    const RBuf b1(a.set1 + (int64_t)s * L.shot_bytes, L.shot_bytes);
    const RBuf bm(a.m.base + (int64_t)s * a.m.shot_stride, a.m.bytes);
    // a stage whose step is not stored gets null destinations: empty views
    const uint32_t sb0 = (SNAP != SNAP_NONE && a.snap0 != nullptr) ? a.snap_shot_bytes : 0u;
    const uint32_t sb1 = (SNAP != SNAP_NONE && a.snap1 != nullptr) ? a.snap_shot_bytes : 0u;
    const int64_t so_s = (int64_t)s * a.snap_shot_bytes;
    const RBuf bsp0(sb0 ? a.snap0 + so_s : nullptr, sb0);
    const RBuf bsp1(sb1 ? a.snap1 + so_s : nullptr, sb1);
    const RBuf bev(a.ev.base, a.ev.bytes);
    const uint32_t c4 = (uint32_t)c * 4u, bx4 = (uint32_t)bxc * 4u;
    const uint32_t rowb = (uint32_t)nx * 4u, brow = (uint32_t)g.bx * 4u;

    // loop-invariant lane offsets of the fast blocks
    const int v_in = lane_off(incol, c4), v_e = lane_off(colE, c4), v_hz = lane_off(colHz, c4);
    const int v_own = lane_off(own, c4), v_ownhz = lane_off(own & colHz, c4);
    const int v_mxh = lane_off(colHz & fx_h, bx4), v_mxe = lane_off(colE & fx_e, bx4);
    const int v_snap = lane_off(own & in_x, (uint32_t)(c - g.x0) * 2u * ESZ);

    const int r_first = ya - 2 * P + 1;
    const int r_end = yb + 4 * P - 3;
    // Unrolled blocks starting at r0 in [f_lo, f_hi] are fast: every stage
    // active, no band row, rows owned / inside the sets, no event row, for
    // all rows the block computes and prefetches (r0 .. r0+U-1+D).
    const int f_lo = max(ya, g.y0) + 4 * P - 2;
    const int f_hi = min(yb + 2 * P - 2, g.hy1 + P - 1) - (U - 1 + D);
    const int e_lo = ev_lo, e_hi = ev_hi;
    // slot of stage-A E row y (ye0 <= y), or -1 (uniform)
    auto slot_of = [&](int y) {
        return (y >= e_lo && y <= e_hi) ? __builtin_amdgcn_readfirstlane(evs[y - ye0]) : -1;
    };

    // Cq of an H row: per-lane offset (negative where masked) + row offset,
    // or a predicate + lane offset (general blocks)
    auto cq_v = [&](int voff, uint32_t soff) {
        if constexpr (UQ) return voff < 0 ? 0.0f : a.cq;
        else return bm.ldv(voff, soff);
    };
    auto cq_p = [&](bool ok, uint32_t off) {
        if constexpr (UQ) return ok ? a.cq : 0.0f;
        else return bm.ld(ok, off, a.m.oCq);
    };

    // Prefetch ring: the loads of iteration r are issued at iteration r - D
    // into slot (r - r_first) % D.
    float fE[D], fQa[D], fHx[D], fHz[D], fMyh[D], fMxh[D], fCa[D], fCb[D], fMxe[D], fMye[D];
    float fQb[D], fCaB[D], fCbB[D], fEvA[D], fEvB[D];
    int fGA[D], fGB[D];                             // slots of rows yA / yB, or -1
    // The loads of a row come in five groups, each issued for row r + D
    // right after the part of row r's iteration that last reads the group's
    // slot: K1 (E, Hx, Myh) after (a), K2 (Cq, Hz, Mxh of stage A) after
    // (b), K3 (stage A's E inputs and events) after (c), K4 (stage B's Cq)
    // after stage B's Hx, K5 (stage B's E inputs and events) at the end.
    auto issue = [&](auto fast_t, auto part_t, int u, int r, bool live) {
        constexpr bool FAST = decltype(fast_t)::value;
        constexpr int K = decltype(part_t)::value;
        const int hA = r - P, yA = r - 2 * P + 1, hB = r - 3 * P + 1, yB = r - 4 * P + 2;
        if constexpr (FAST) {
            const uint32_t rA = (uint32_t)hA * rowb, eA = (uint32_t)yA * rowb;
            if constexpr (K == 1) {
                fE[u] = b0.ldv(v_in, L.oE + (uint32_t)r * rowb);
                fHx[u] = b0.ldv(v_e, L.oHx + rA);
            } else if constexpr (K == 2) {
                fQa[u] = cq_v(v_in, a.m.oCq + rA);
                fHz[u] = b0.ldv(v_hz, L.oHz + rA);
                fMxh[u] = b0.ldv(xband ? v_mxh : RBuf::OOB, L.oMxh + (uint32_t)hA * brow);
            } else if constexpr (K == 3) {
                fGA[u] = -1;
                fCa[u] = bm.ldv(v_e, a.m.oCa + eA);
                fCb[u] = bm.ldv(v_e, a.m.oCb + eA);
                fMxe[u] = b0.ldv(xband ? v_mxe : RBuf::OOB, L.oMxe + (uint32_t)yA * brow);
            } else if constexpr (K == 4) {
                fQb[u] = cq_v(v_in, a.m.oCq + (uint32_t)hB * rowb);
            } else {
                fGB[u] = -1;
                fCaB[u] = bm.ldv(v_own, a.m.oCa + (uint32_t)yB * rowb);
                fCbB[u] = bm.ldv(v_own, a.m.oCb + (uint32_t)yB * rowb);
            }
        } else {
            const uint32_t ohA = (uint32_t)(hA * nx) * 4u + c4, oyA = (uint32_t)(yA * nx) * 4u + c4;
            const uint32_t ohB = (uint32_t)(hB * nx) * 4u + c4, oyB = (uint32_t)(yB * nx) * 4u + c4;
            if constexpr (K == 1) {
                fE[u] = b0.ld(live & in_rows(r) & incol, (uint32_t)(r * nx) * 4u + c4, L.oE);
                const bool hx_do = live & colE & hx_row(hA);
                fHx[u] = b0.ld(hx_do, ohA, L.oHx);
                fMyh[u] = b0.ld(hx_do & fy_h(hA), (uint32_t)(band_y(g, hA) * nx) * 4u + c4, L.oMyh);
            } else if constexpr (K == 2) {
                fQa[u] = cq_p(live & in_rows(hA) & incol, ohA);
                const bool hz_do = live & colHz & hz_row(hA) & (hA >= ye0) & (hA <= yb + 2 * P - 2);
                fHz[u] = b0.ld(hz_do, ohA, L.oHz);
                fMxh[u] = b0.ld(hz_do & fx_h, (uint32_t)(hA * g.bx) * 4u + bx4, L.oMxh);
            } else if constexpr (K == 3) {
                // event row first (uniform branch), then the loads every row has
                const int gA = slot_of(yA);
                fGA[u] = gA;
                fEvA[u] = 0.0f;
                if (gA >= 0) fEvA[u] = bev.ld(live & incol, (uint32_t)(gA * nx) * 4u + c4, a.es0.add);
                const bool e_do = live & colE & rowE(yA) & (yA >= ye0);
                fCa[u] = bm.ld(e_do, oyA, a.m.oCa);
                fCb[u] = bm.ld(e_do, oyA, a.m.oCb);
                fMxe[u] = b0.ld(e_do & fx_e, (uint32_t)(yA * g.bx) * 4u + bx4, L.oMxe);
                fMye[u] = b0.ld(e_do & fy_e(yA), (uint32_t)(band_y(g, yA) * nx) * 4u + c4, L.oMye);
            } else if constexpr (K == 4) {
                fQb[u] = cq_p(live & in_rows(hB) & incol & (hB >= ya - P), ohB);
            } else {
                const bool eb_do = live & own & own_row(yB);
                const int gB = slot_of(yB);
                fGB[u] = gB;
                fEvB[u] = 0.0f;
                if (gB >= 0) fEvB[u] = bev.ld(eb_do, (uint32_t)(gB * nx) * 4u + c4, a.es1.add);
                fCaB[u] = bm.ld(eb_do, oyB, a.m.oCa);
                fCbB[u] = bm.ld(eb_do, oyB, a.m.oCb);
            }
        }
    };
    using K1 = std::integral_constant<int, 1>;
    using K2 = std::integral_constant<int, 2>;
    using K3 = std::integral_constant<int, 3>;
    using K4 = std::integral_constant<int, 4>;
    using K5 = std::integral_constant<int, 5>;

    float ewA[2 * P];    // E^n rows r-2P+1 .. r
    float hwA[2 * P];    // Hx^{n+1/2} rows hA-2P+1 .. hA
    float ewB[2 * P];    // E^{n+1} rows yA-2P+1 .. yA
    float hwB[2 * P];    // Hx^{n+3/2} rows hB-2P+1 .. hB
#pragma unroll
    for (int i = 0; i < 2 * P; ++i) { ewA[i] = 0.0f; hwA[i] = 0.0f; ewB[i] = 0.0f; hwB[i] = 0.0f; }
#pragma unroll
    for (int i = 1; i < 2 * P; ++i) {
        const int r = r_first - 2 * P + i;
        ewA[i] = b0.ld(in_rows(r) & incol, (uint32_t)(r * nx) * 4u + c4, L.oE);
    }
#pragma unroll
    for (int u = 0; u < D; ++u) {
        const int r = r_first + u;
        issue(std::false_type{}, K1{}, u, r, r <= r_end);
        issue(std::false_type{}, K2{}, u, r, r <= r_end);
        issue(std::false_type{}, K3{}, u, r, r <= r_end);
        issue(std::false_type{}, K4{}, u, r, r <= r_end);
        issue(std::false_type{}, K5{}, u, r, r <= r_end);
    }

    // One iteration (row r, prefetch slot u).  FAST: the block is fast (all
    // row predicates true / false as described above).  The loads of row
    // rn = r + D (liveness live_n) go into slot u as the iteration frees it.
    auto iter = [&](auto fast_t, int r, int u, int rn, bool live_n) {
        constexpr bool FAST = decltype(fast_t)::value;
        const int hA = r - P, yA = r - 2 * P + 1, hB = r - 3 * P + 1, yB = r - 4 * P + 2;

        // ---- (a) new E^n row; LDS rows for the two Hz stencils; Hx of stage A
#pragma unroll
        for (int i = 0; i < 2 * P - 1; ++i) ewA[i] = ewA[i + 1];
        ewA[2 * P - 1] = fE[u];
        float* const rA = rowA[r & 1];
        float* const rB = rowB[r & 1];
        rA[tid] = ewA[P - 1];
        rB[tid] = ewB[P];
        {
            float d = g.rdy * stencil<P>([&](int k) { return ewA[P - 1 + k]; },
                                         [&](int k) { return ewA[P - k]; });
            if (!FAST && fy_h(hA)) {                                    // uniform
                const float* ct = cyt[hA - yc0];
                float m = fMyh[u];
                d = cpml_step(m, ct[0], ct[1], ct[2], d);
                yref(0, slot2(hA)) = m;
            }
            const bool hx_ok = FAST ? colE : (colE & hx_row(hA));
            const float hxn = hx_ok ? fmaf(-fQa[u], d, fHx[u]) : 0.0f;
#pragma unroll
            for (int i = 0; i < 2 * P - 1; ++i) hwA[i] = hwA[i + 1];
            hwA[2 * P - 1] = hxn;
        }
        issue(fast_t, K1{}, u, rn, live_n);
        __syncthreads();

        // ---- (b) Hz of stage A (row hA) and of stage B (row hB)
        if (FAST || (hz_row(hA) & (hA >= ye0) & (hA <= yb + 2 * P - 2))) {   // uniform
            float d = g.rdx * stencil<P>([&](int k) { return rA[th + k]; },
                                         [&](int k) { return rA[th - k + 1]; });
            if (xband) {
                float m = fMxh[u];
                d = cpml_step(m, cx_h.a, cx_h.b, cx_h.ik, d);
                xput(0, slot2(hA), m);
            }
            ringA[slot2(hA)][tid] = hzA_ok ? fmaf(fQa[u], d, fHz[u]) : 0.0f;
        }
        if (FAST || (hz_row(hB) & own_row(hB))) {                             // uniform
            float d = g.rdx * stencil<P>([&](int k) { return rB[th + k]; },
                                         [&](int k) { return rB[th - k + 1]; });
            if (xband) {
                float m = xget(0, slot2(hB));
                d = cpml_step(m, cx_h.a, cx_h.b, cx_h.ik, d);
                if constexpr (FAST) b1.stv(m, lane_off(own & colHz & fx_h, bx4), L.oMxh + (uint32_t)hB * brow);
                else b1.st(own & colHz & fx_h, m, (uint32_t)(hB * g.bx) * 4u + bx4, L.oMxh);
            }
            const float hzn = hzB_ok ? fmaf(fQb[u], d, ringA[slot2(hB)][tid]) : 0.0f;
            if constexpr (FAST) b1.stv(hzn, v_ownhz, L.oHz + (uint32_t)hB * rowb);
            else b1.st(own & colHz, hzn, (uint32_t)(hB * nx) * 4u + c4, L.oHz);
            ringB[slot1(hB)][tid] = hzn;
        }
        issue(fast_t, K2{}, u, rn, live_n);
        // P >= 2: both E rows read ring rows written P-1 rows earlier and the
        // row buffers alternate, so one barrier per row suffices
        if constexpr (P == 1) __syncthreads();

        // ---- (c) E of stage A (row yA), with the step-n sources and receivers
        if (FAST || r >= ya) {                                                // uniform
            const float* hzr = ringA[slot2(yA)];
            float uu_ = g.rdx * stencil<P>([&](int k) { return hzr[te + k - 1]; },
                                           [&](int k) { return hzr[te - k]; });
            if (xband) {
                float m = fMxe[u];
                uu_ = cpml_step(m, cx_e.a, cx_e.b, cx_e.ik, uu_);
                xput(1, slot2(yA), m);
            }
            float v = g.rdy * stencil<P>([&](int k) { return hwA[P - 1 + k]; },
                                         [&](int k) { return hwA[P - k]; });
            if (!FAST && fy_e(yA)) {
                const float* ct = cyt[yA - yc0];
                float m = fMye[u];
                v = cpml_step(m, ct[3], ct[4], ct[5], v);
                yref(1, slot2(yA)) = m;
            }
            const float curl = uu_ - v;
            const float ev = ewA[0];
            if constexpr (SNAP != SNAP_NONE) {
                if constexpr (FAST) {
                    const uint32_t so = (uint32_t)((yA - g.y0) * g.nxi) * 2u * ESZ;
                    snap_put2v<SNAP>(bsp0, ev, curl, v_snap, so);
                } else if ((yA >= g.y0) & (yA < g.y1) & own_row(yA)) {
                    const uint32_t w = (uint32_t)((yA - g.y0) * g.nxi + (c - g.x0));
                    snap_put2<SNAP>(bsp0, own & in_x, w, ev, curl);
                }
            }
            float en = fmaf(fCa[u], ev, fCb[u] * curl);
            en = (FAST ? eA_ok : (eA_ok & rowE(yA))) ? en : 0.0f;
            if (!FAST && fGA[u] >= 0) {                                  // uniform
                en = en + fEvA[u];
                bev.st(own & own_row(yA), en, (uint32_t)(fGA[u] * nx) * 4u + c4, a.es0.out);
            }
#pragma unroll
            for (int i = 0; i < 2 * P - 1; ++i) ewB[i] = ewB[i + 1];
            ewB[2 * P - 1] = en;
        }
        issue(fast_t, K3{}, u, rn, live_n);

        // ---- Hx of stage B (row hB)
        if (FAST || r >= ya + 2 * P - 1) {                                    // uniform
            float d = g.rdy * stencil<P>([&](int k) { return ewB[P - 1 + k]; },
                                         [&](int k) { return ewB[P - k]; });
            const bool st_h = FAST ? own : (own & hx_row(hB) & own_row(hB));
            if (!FAST && fy_h(hB)) {
                const float* ct = cyt[hB - yc0];
                float m = yref(0, slot2(hB));
                d = cpml_step(m, ct[0], ct[1], ct[2], d);
                b1.st(st_h, m, (uint32_t)(band_y(g, hB) * nx) * 4u + c4, L.oMyh);
            }
            const bool hx_ok = FAST ? colE : (colE & hx_row(hB));
            const float hxn = hx_ok ? fmaf(-fQb[u], d, hwA[0]) : 0.0f;
            if constexpr (FAST) b1.stv(hxn, v_own, L.oHx + (uint32_t)hB * rowb);
            else b1.st(st_h, hxn, (uint32_t)(hB * nx) * 4u + c4, L.oHx);
#pragma unroll
            for (int i = 0; i < 2 * P - 1; ++i) hwB[i] = hwB[i + 1];
            hwB[2 * P - 1] = hxn;
        }
        issue(fast_t, K4{}, u, rn, live_n);

        // ---- E of stage B (row yB): the owned output row
        if (FAST || r >= ya + 4 * P - 2) {                                    // uniform
            const float* hzr = ringB[slot1(yB)];
            float uu_ = g.rdx * stencil<P>([&](int k) { return hzr[te + k - 1]; },
                                           [&](int k) { return hzr[te - k]; });
            if (xband) {
                float m = xget(1, slot2(yB));
                uu_ = cpml_step(m, cx_e.a, cx_e.b, cx_e.ik, uu_);
                if constexpr (FAST) b1.stv(m, lane_off(own & fx_e, bx4), L.oMxe + (uint32_t)yB * brow);
                else b1.st(own & fx_e, m, (uint32_t)(yB * g.bx) * 4u + bx4, L.oMxe);
            }
            float v = g.rdy * stencil<P>([&](int k) { return hwB[P - 1 + k]; },
                                         [&](int k) { return hwB[P - k]; });
            if (!FAST && fy_e(yB)) {
                const float* ct = cyt[yB - yc0];
                float m = yref(1, slot2(yB));
                v = cpml_step(m, ct[3], ct[4], ct[5], v);
                b1.st(own, m, (uint32_t)(band_y(g, yB) * nx) * 4u + c4, L.oMye);
            }
            const float curl = uu_ - v;
            const float ev = ewB[0];
            if constexpr (SNAP != SNAP_NONE) {
                if constexpr (FAST) {
                    const uint32_t so = (uint32_t)((yB - g.y0) * g.nxi) * 2u * ESZ;
                    snap_put2v<SNAP>(bsp1, ev, curl, v_snap, so);
                } else if ((yB >= g.y0) & (yB < g.y1)) {
                    const uint32_t w = (uint32_t)((yB - g.y0) * g.nxi + (c - g.x0));
                    snap_put2<SNAP>(bsp1, own & in_x, w, ev, curl);
                }
            }
            float en = fmaf(fCaB[u], ev, fCbB[u] * curl);
            if constexpr (FAST) {
                b1.stv(en, v_own, L.oE + (uint32_t)yB * rowb);
            } else {
                if (fGB[u] >= 0) {                                      // uniform
                    en = en + fEvB[u];
                    bev.st(own, en, (uint32_t)(fGB[u] * nx) * 4u + c4, a.es1.out);
                }
                b1.st(own, en, (uint32_t)(yB * nx) * 4u + c4, L.oE);
            }
        }
        issue(fast_t, K5{}, u, rn, live_n);
    };

    for (int r0 = r_first;; r0 += U) {
        // uniform: all rows this block computes and prefetches are steady
        const bool fast = r0 >= f_lo && r0 <= f_hi &&
                          (r0 + U + D - 2 * P < e_lo || r0 - 4 * P + 2 > e_hi);
        if (fast) {
#pragma unroll
            for (int uu = 0; uu < U; ++uu) {
                iter(std::true_type{}, r0 + uu, uu % D, r0 + uu + D, true);
            }
        } else {
#pragma unroll
            for (int uu = 0; uu < U; ++uu) {
                const int r = r0 + uu;
                if (r > r_end) return;
                iter(std::false_type{}, r, uu % D, r + D, r + D <= r_end);
            }
        }
    }
}

}  // namespace tmf
