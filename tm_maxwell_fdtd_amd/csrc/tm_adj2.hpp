// Two adjoint time steps per launch (temporal blocking), gfx950 / wave64.
//
// k_adj_step2 takes the adjoint state from after step n+1 back to after
// step n-1 in one pass over the state: stage A is the adjoint step n exactly
// as k_adj_step computes it, stage B the adjoint step n-1, fed by stage A's
// rows while they are still on chip.  The state crosses HBM once per two
// steps and the per-shot gradients are read and written once: at a row,
// both steps' gradient terms are added in the order two single steps add
// them (step n's first), so both paths give bitwise the same gradients.
//
// Streaming (iteration r; stage B runs 2P rows behind stage A):
//   stage A: input row r,       H row hA = r - P,   E row yA = r - 2P + 1
//   stage B: input row rB = r - 2P,  hB = rB - P,   yB = rB - 2P + 1
// Stage B's input lambda_E^n(rB) is stage A's E row of the previous
// iteration (one register); the old lambda_Hx^n, lambda_Hz^n of row hB are
// stage A's H rows of 2P iterations before (per-lane register windows);
// stage A's updated CPML memories wait 2P iterations in lane-private LDS
// FIFOs.  Within an iteration stage B goes first, so it reads a window or
// FIFO slot before stage A overwrites it, and the two stages share the two
// barriers of the iteration.  The gradients of row rB use lambda_E^{n+1}(rB)
// still in stage A's register window and stage B's input lambda_E^n(rB).
//
// A strip of 256 lanes owns up to W = 256 - 8P + 4 columns (the strips of
// a grid are cut to equal widths, Tiling::W): stage A's lambda_E is
// valid 2P-1 lanes in from the edges, stage B's another 2P-1; a chunk of CH
// owned rows reads 4P-2 rows above and 4P-1 below.  Stage A's values
// outside the fields' index sets are forced to 0, as the cells the single
// step never writes stay 0.
#pragma once

#include "tm_step.hpp"
#include "tm_step2.hpp"

namespace tmf {

constexpr int CHA2_MAX = 160;   // largest chunk height of the two-step adjoint (LDS tables)
constexpr int PREFETCH_A2 = 1;  // rows of loads in flight ahead (one iteration covers both stages)
constexpr int UNROLL_A2 = 2;    // row-loop unroll

struct Adj2Args {
    Geo g;
    Tiling t;
    StateLayout L;
    Model m;
    const float* __restrict__ cp;
    const char* __restrict__ set0;     // adjoint state after step n+1
    char* __restrict__ set1;           // adjoint state after step n-1
    const char* __restrict__ snapA;    // (Ey^n, curl H^n) pairs [S][nyi][nxi][2], or null (step n not stored)
    const char* __restrict__ snapB;    // (Ey^{n-1}, curl H^{n-1}) pairs, or null
    uint32_t snap_shot_bytes;          // bytes of one shot's pairs
    float* __restrict__ gca;           // per-shot gradients [S][ny][nx], or null
    float* __restrict__ gcb;
    float ratio;                       // weight of a stored step's gradient term
    EventRows ev;                      // residual at the receivers (add), sources (out)
    EventStep esA, esB;                // ... of steps n and n-1
    float cq;                          // Cq where it holds one value (UQ instances)
};

// UQ: Cq holds one value (mu_r uniform), passed as cq: no Cq bytes are read,
// and each Cq load becomes that value where the load would have read a cell
// (0 where it is masked), bitwise what the array gives.
template <int P, int SNAP, bool UQ>
__global__ __launch_bounds__(NT, P == 2 ? 4 : 3) void k_adj_step2(Adj2Args a)
{
    constexpr int OFF = Strip2<P>::OFF;
    constexpr int D = PREFETCH_A2;
    constexpr int R2 = 2 * P;                       // window / FIFO depth (a power of two)
    constexpr uint32_t ESZ = snap_bytes<SNAP>();
    constexpr int GRAD_PART = P == 4 ? 1 : 3;       // load group of stage B's gradients and snapshots
    __shared__ float rowUA[NT], rowUB[NT];          // u of rows hA / hB (x-stencils of lambda_Hz)
    __shared__ float ringA[P][NT], ringB[P][NT];    // filtered Cq lambda_Hz rows of each stage
    __shared__ float mfifo[4][R2][NT];              // stage A's Mxe, Mye, Myh, Mxh, lane-private
    __shared__ float cyt[CHA2_MAX + 8 * P][6];      // per-row CPML coefficients
    __shared__ int evs[CHA2_MAX + 8 * P];           // row slots of the event rows
    __shared__ int ev_lo, ev_hi;

    const Geo& g = a.g;
    const StateLayout& L = a.L;
    int s, strip, ya, yb;
    tile2_of(a.t, g.ny, P, s, strip, ya, yb);
    const int tid = threadIdx.x;
    const int nx = g.nx, ny = g.ny;
    const int xs = P + strip * a.t.W;               // a.t.W <= Strip2<P>::W
    const int xe = min(xs + a.t.W, nx - P + 1);
    const int Ya = ya - 2 * P + 1, Yb = yb + 2 * P - 1;   // stage A's output rows [Ya, Yb)
    const int yt = ya - 4 * P + 2;                  // first row of the tables (stage A's first input row)
    const int r_end = yb + 4 * P - 2;               // last iteration (stage B's last input row + 2P)
    if (tid == 0) {
        ev_lo = INT32_MAX;
        ev_hi = INT32_MIN;
    }
    __syncthreads();
    load_row_cpml(cyt, a.cp, g, yt, r_end - yt + 1);
    load_row_slots(evs, &ev_lo, &ev_hi, a.ev.row_slot, s, ny, yt, r_end - yt + 1);
    __syncthreads();
    const int e_lo = ev_lo, e_hi = ev_hi;

    const int c = xs - OFF + tid;
    const bool own = (c >= xs) & (c < xe);
    const bool colE = (c >= P) & (c <= nx - P);
    const bool colHz = (c >= P) & (c <= nx - P - 1);
    const bool hzA_ok = colHz & (tid >= P - 1) & (tid <= NT - P - 1);        // stage A lambda_Hz lanes
    const bool eA_ok = colE & (tid >= 2 * P - 1) & (tid <= NT - 2 * P);     // stage A lambda_E lanes
    const bool hzB_ok = colHz & (tid >= 3 * P - 2) & (tid <= NT - 3 * P);   // stage B lambda_Hz lanes
    const bool fx_h = colE & ((c < g.x0) | (c >= g.hx1));
    const bool fx_e = colE & ((c < g.x0) | (c >= g.x1));
    const bool in_x = (c >= g.x0) & (c < g.x1);
    const int c0 = xs - OFF;
    const bool xband = c0 < g.x0 || c0 + NT - 1 >= g.hx1;   // uniform
    const int bxc = band_x(g, (c >= 0 && c < nx) ? c : 0);
    const int th = min(max(tid, P - 1), NT - P - 1);
    const int te = min(max(tid, P), NT - P);
    const bool grad = SNAP != SNAP_NONE && own && in_x;

    Cpml1 cx_h{0.f, 0.f, 1.f}, cx_e{0.f, 0.f, 1.f};
    if (fx_h) cx_h = cpml_at(a.cp, g.L, AXH, c);
    if (fx_e) cx_e = cpml_at(a.cp, g.L, AX, c);

    auto e_row = [&](int r) { return (r >= P) & (r <= ny - P); };
    auto hx_row = [&](int h) { return (h >= P) & (h <= ny - P - 1); };
    auto own_row = [&](int y) { return (y >= ya) & (y < yb); };
    auto hzA_row = [&](int h) { return (h >= Ya) & (h < Yb) & (h >= P) & (h <= ny - P); };
    auto hzB_row = [&](int h) { return own_row(h) & (h >= P) & (h <= ny - P); };
    auto fy_h = [&](int h) { return (h < g.y0) | (h >= g.hy1); };
    auto fy_e = [&](int y) { return (y < g.y0) | (y >= g.y1); };
    auto fslot = [&](int y) { return (y + 4 * P) & (R2 - 1); };   // y >= -3P

    const RBuf b0(a.set0 + (int64_t)s * L.shot_bytes, L.shot_bytes);
    const RBuf b1(a.set1 + (int64_t)s * L.shot_bytes, L.shot_bytes);
    const RBuf bm(a.m.base + (int64_t)s * a.m.shot_stride, a.m.bytes);
    const uint32_t sbA = (SNAP != SNAP_NONE && a.snapA != nullptr) ? a.snap_shot_bytes : 0u;
    const uint32_t sbB = (SNAP != SNAP_NONE && a.snapB != nullptr) ? a.snap_shot_bytes : 0u;
    const int64_t so_s = (int64_t)s * a.snap_shot_bytes;
    const RBuf bspA(sbA ? a.snapA + so_s : nullptr, sbA), bspB(sbB ? a.snapB + so_s : nullptr, sbB);
    const uint32_t slab_b = (uint32_t)(g.slab * 4);
    const RBuf bga(a.gca + (int64_t)s * g.slab, a.gca ? slab_b : 0u);
    const RBuf bgb(a.gcb + (int64_t)s * g.slab, a.gcb ? slab_b : 0u);
    const RBuf bev(a.ev.base, a.ev.bytes);
    const uint32_t c4 = (uint32_t)c * 4u, bx4 = (uint32_t)bxc * 4u;
    const uint32_t rowb = (uint32_t)nx * 4u, brow = (uint32_t)g.bx * 4u;

    // Addressing as in k_adj_step: loop-invariant lane offsets (out of range
    // where the lane never touches the array), per-row masks, clamped rows.
    const int v_e = lane_off(colE, c4), v_own = lane_off(own, c4), v_eA = lane_off(eA_ok, c4);
    const int v_hz = lane_off(hzA_ok, c4), v_hzo = lane_off(colHz, c4);
    const int v_xe = lane_off(fx_e, bx4);
    const int v_hzxh = lane_off(hzA_ok & fx_h, bx4), v_hzxo = lane_off(colHz & fx_h, bx4);
    // v | the OOB bit of the non-owned columns, rebuilt at each use (the
    // empty asm keeps it inside the row loop) so that the owned-column
    // variants of the offsets take no registers of their own.
    auto ownv = [&](int v) {
        int o = v_own;
        asm volatile("" : "+v"(o));
        return v | (o & RBuf::OOB);
    };
    const int v_g = lane_off(grad, c4), v_gs = lane_off(grad, (uint32_t)(c - g.x0) * 2u * ESZ);
    auto msk = [](bool ok) { return ok ? 0 : RBuf::OOB; };
    // ring slot of a row; at order 4 the slot is the row's parity, fixed in
    // each unrolled iteration, and the empty asm makes the compiler rebuild
    // the slot's LDS address at each use instead of holding (or spilling)
    // one address per slot
    auto rslot = [](int s) {
        if constexpr (P == 2) asm volatile("" : "+s"(s));
        return s;
    };
    auto grow = [&](int y) { return (uint32_t)min(max(y, 0), ny - 1); };
    auto brw = [&](int y) { return (uint32_t)min(max(band_y(g, y), 0), g.by - 1); };
    auto srw = [&](int y) { return (uint32_t)min(max(y - g.y0, 0), g.nyi - 1) * (uint32_t)g.nxi * 2u * ESZ; };
    auto slot_of = [&](int y) {
        return (y >= e_lo && y <= e_hi) ? __builtin_amdgcn_readfirstlane(evs[y - yt]) : -1;
    };
    auto ctab = [&](int y) { return cyt[y - yt]; };

    // Prefetch ring: the loads of iteration r are issued at iteration r - D.
    // FAST: every row the iteration touches is active, owned, inside the
    // index sets, off the y bands and free of events (see the block test
    // below), so the row masks and clamps fold away.
    float fE[D], fCbA[D], fMxe[D], fMye[D], fHx[D], fMyh[D], fQA[D], fHz[D], fMxh[D], fCaA[D], fEvA[D];
    float fCbB[D], fSeA[D], fScA[D], fSeB[D], fScB[D], fGa[D], fGb[D], fQB[D], fCaB[D], fEvB[D];
    int fGA[D], fGB[D];
    // The loads of a row come in three groups, each issued for the next row
    // as soon as the current row's iteration has used that group's slots, so
    // that most loads get nearly a whole iteration of lead: PART 1 (fronts'
    // inputs and stage A's lambda_Hx inputs) after phase 1, PART 2 (Cq and
    // the lambda_Hz inputs) after phase 2, PART 3 (Ca) after phase 3.  The
    // gradient accumulators and snapshots of stage B's front, read in phase
    // 1, go with PART 1 at order 8 (a whole iteration of lead within the
    // register budget) and with PART 3 at lower orders (a short lead, which
    // keeps their registers free across phases 2 and 3).
    auto issue = [&](auto fast_t, auto part_t, int u, int r, bool live) {
        constexpr bool FAST = decltype(fast_t)::value;
        constexpr int PART = decltype(part_t)::value;
        auto M = [&](bool ok) { return FAST ? 0 : msk(ok); };
        auto G = [&](int y) { return FAST ? (uint32_t)y : grow(y); };
        const int hA = r - P, yA = r - 2 * P + 1, rB = r - 2 * P, hB = rB - P, yB = rB - 2 * P + 1;
        const bool liveA = live & (r <= r_end - 1);
        const bool liveB = live & (r >= ya + 1);
        const int meA = M(liveA & e_row(r)), meB = M(liveB & e_row(rB));
        if constexpr (PART == GRAD_PART) {
            const uint32_t orB = G(rB) * rowb;
            const int mg = M(liveB & own_row(rB) & (rB >= g.y0) & (rB < g.y1));
            const uint32_t sr = FAST ? (uint32_t)(rB - g.y0) * (uint32_t)g.nxi * 2u * ESZ : srw(rB);
            const SnapPair pA = snap_get2v<SNAP>(bspA, v_gs | mg, sr);
            const SnapPair pB = snap_get2v<SNAP>(bspB, v_gs | mg, sr);
            fSeA[u] = pA.e;
            fScA[u] = pA.c;
            fSeB[u] = pB.e;
            fScB[u] = pB.c;
            fGa[u] = bga.ldv(v_g | mg, orB);
            fGb[u] = bgb.ldv(v_g | mg, orB);
        }
        if constexpr (PART == 3) {
            fCaA[u] = bm.ldv(v_eA | M(liveA & (yA >= Ya) & (yA < Yb) & e_row(yA)), a.m.oCa + G(yA) * rowb);
            fCaB[u] = bm.ldv(v_own | M(liveB & own_row(yB)), a.m.oCa + G(yB) * rowb);
            return;
        }
        if constexpr (PART == 2) {
            const uint32_t ohA = G(hA) * rowb;
            if constexpr (UQ) {
                const int qo = v_e | M(liveA & (hx_row(hA) | hzA_row(hA)));
                fQA[u] = qo < 0 ? 0.0f : a.cq;
            } else {
                fQA[u] = bm.ldv(v_e | M(liveA & (hx_row(hA) | hzA_row(hA))), a.m.oCq + ohA);
            }
            const int mzA = M(liveA & hzA_row(hA));
            fHz[u] = b0.ldv(v_hz | mzA, L.oHz + ohA);
            fMxh[u] = b0.ldv(xband ? (v_hzxh | mzA) : RBuf::OOB, L.oMxh + G(hA) * brow);
            if constexpr (UQ) {
                const int qo = v_e | M(liveB & (hx_row(hB) | own_row(hB)));
                fQB[u] = qo < 0 ? 0.0f : a.cq;
            } else {
                fQB[u] = bm.ldv(v_e | M(liveB & (hx_row(hB) | own_row(hB))), a.m.oCq + G(hB) * rowb);
            }
            return;
        }
        if constexpr (FAST) {
            fGA[u] = -1;
            fGB[u] = -1;
        } else {
            const int gA = slot_of(r), gB = slot_of(rB);
            fGA[u] = gA;
            fGB[u] = gB;
            fEvA[u] = 0.0f;
            fEvB[u] = 0.0f;
            if (gA >= 0) fEvA[u] = bev.ldv(v_e | meA, (uint32_t)gA * rowb + a.esA.add);   // uniform
            if (gB >= 0) fEvB[u] = bev.ldv(v_e | meB, (uint32_t)gB * rowb + a.esB.add);
        }
        // stage A
        const uint32_t orA = G(r) * rowb, ohA = G(hA) * rowb;
        fE[u] = b0.ldv(v_e | meA, L.oE + orA);
        fCbA[u] = bm.ldv(v_e | meA, a.m.oCb + orA);
        fMxe[u] = b0.ldv(xband ? (v_xe | meA) : RBuf::OOB, L.oMxe + G(r) * brow);
        const int mhA = M(liveA & hx_row(hA));
        fHx[u] = b0.ldv(v_e | mhA, L.oHx + ohA);
        if constexpr (!FAST) {                            // y-band memories (never on fast rows)
            fMye[u] = b0.ldv(v_e | meA | msk(fy_e(r)), L.oMye + brw(r) * rowb);
            fMyh[u] = b0.ldv(v_e | mhA | msk(fy_h(hA)), L.oMyh + brw(hA) * rowb);
        }
        // stage B
        const uint32_t orB = G(rB) * rowb;
        fCbB[u] = bm.ldv(v_e | meB, a.m.oCb + orB);
    };
    using Part1 = std::integral_constant<int, 1>;
    using Part2 = std::integral_constant<int, 2>;
    using Part3 = std::integral_constant<int, 3>;

    float edA[R2], wwA[R2], twA[R2], udA[P + 1];   // as ed, ww, tw, ud of k_adj_step, stage A
    float edB[R2], wwB[R2], twB[R2], udB[P + 1];   // ... stage B
    float hxA[R2], hzA[R2];                        // stage A's lambda_Hx^n, lambda_Hz^n, rows hA-2P .. hA-1
    float eAprev = 0.0f;                           // stage A's lambda_E^n of row r-2P (stage B's input)
#pragma unroll
    for (int i = 0; i < R2; ++i) {
        edA[i] = 0.0f; wwA[i] = 0.0f; twA[i] = 0.0f; edB[i] = 0.0f; wwB[i] = 0.0f; twB[i] = 0.0f;
        hxA[i] = 0.0f; hzA[i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i <= P; ++i) { udA[i] = 0.0f; udB[i] = 0.0f; }

    auto push = [&](float (&ed)[R2], float (&ww)[R2], float (&ud)[P + 1], float e, float u, float w) {
#pragma unroll
        for (int i = 0; i < R2 - 1; ++i) { ed[i] = ed[i + 1]; ww[i] = ww[i + 1]; }
        ed[R2 - 1] = e;
        ww[R2 - 1] = w;
#pragma unroll
        for (int i = 0; i < P; ++i) ud[i] = ud[i + 1];
        ud[P] = u;
    };
    auto shift_in = [&](float (&win)[R2], float v) {
#pragma unroll
        for (int i = 0; i < R2 - 1; ++i) win[i] = win[i + 1];
        win[R2 - 1] = v;
    };
    // Stage A's front of input row r: lambda_E^{n+1} with the step-n
    // residual added; u, w; the updated memories go to the FIFOs.
    auto frontA = [&](auto fast_t, int r, int gs, float ev, float e, float cbv, float mx, float my) {
        constexpr bool FAST = decltype(fast_t)::value;
        if (!FAST && gs >= 0) {                                           // uniform
            e = e + ev;
            bev.stv(e, v_own | msk(own_row(r)), (uint32_t)gs * rowb + a.esA.out);
        }
        const float hv = cbv * e;
        float u = hv, w = hv;
        if (xband) {
            float m = mx;
            u = cpml_step(m, cx_e.a, cx_e.b, cx_e.ik, hv);
            mfifo[0][fslot(r)][tid] = m;
        }
        if (!FAST && fy_e(r)) {                                           // uniform
            const float* ct = ctab(r);
            float m = my;
            w = cpml_step(m, ct[3], ct[4], ct[5], hv);
            mfifo[1][fslot(r)][tid] = m;
        }
        push(edA, wwA, udA, e, u, w);
    };

    // stage A prologue: input rows yt .. Ya-1 (front only)
    for (int r = yt; r < Ya; ++r) {
        const int me = msk(e_row(r));
        const uint32_t orr = grow(r) * rowb;
        const int gs = slot_of(r);
        float ev = 0.0f;
        if (gs >= 0) ev = bev.ldv(v_e | me, (uint32_t)gs * rowb + a.esA.add);   // uniform
        frontA(std::false_type{}, r, gs, ev, b0.ldv(v_e | me, L.oE + orr), bm.ldv(v_e | me, a.m.oCb + orr),
               b0.ldv(v_xe | me, L.oMxe + grow(r) * brow), b0.ldv(v_e | me | msk(fy_e(r)), L.oMye + brw(r) * rowb));
    }
#pragma unroll
    for (int u = 0; u < D; ++u) {
        issue(std::false_type{}, Part1{}, u, Ya + u, Ya + u <= r_end);
        issue(std::false_type{}, Part2{}, u, Ya + u, Ya + u <= r_end);
        issue(std::false_type{}, Part3{}, u, Ya + u, Ya + u <= r_end);
    }

    // nfast_t / rn / live_n: the issue instance, row and liveness of the
    // next row's loads.
    auto iter = [&](auto fast_t, auto nfast_t, int r, int u, int rn, bool live_n) {
        constexpr bool FAST = decltype(fast_t)::value;
        auto M = [&](bool ok) { return FAST ? 0 : msk(ok); };
        auto G = [&](int y) { return FAST ? (uint32_t)y : grow(y); };
        const int hA = r - P, yA = r - 2 * P + 1, rB = r - 2 * P, hB = rB - P, yB = rB - 2 * P + 1;
        const bool actA = FAST || r <= r_end - 1;         // uniform
        const bool actB = FAST || r >= ya + 1;            // stage B has input rows
        const bool fullB = FAST || r >= ya + 2 * P;       // ... and H rows

        // ---- phase 1: fronts, gradients, lambda_Hx of both stages
        if (actB) {                                       // stage B front of row rB (uniform)
            float e = eAprev;
            const int gs = fGB[u];
            if (!FAST && gs >= 0) {                       // uniform
                e = e + fEvB[u];
                bev.stv(e, v_own | msk(own_row(rB)), (uint32_t)gs * rowb + a.esB.out);
            }
            if constexpr (SNAP != SNAP_NONE) {
                if (FAST || (own_row(rB) & (rB >= g.y0) & (rB < g.y1))) {   // uniform
                    const uint32_t orr = (uint32_t)rB * rowb;
                    const float eA = edA[0];              // lambda_E^{n+1}(rB) with step n's residual
                    float ga = fGa[u], gb = fGb[u];
                    if (sbA) { ga = fmaf(eA, fSeA[u] * a.ratio, ga); gb = fmaf(eA, fScA[u] * a.ratio, gb); }
                    if (sbB) { ga = fmaf(e, fSeB[u] * a.ratio, ga); gb = fmaf(e, fScB[u] * a.ratio, gb); }
                    bga.stv(ga, v_g, orr);
                    bgb.stv(gb, v_g, orr);
                }
            }
            const int ms = M(own_row(rB) & e_row(rB));
            const float hv = fCbB[u] * e;
            float uu = hv, w = hv;
            if (xband) {
                float m = mfifo[0][fslot(rB)][tid];
                uu = cpml_step(m, cx_e.a, cx_e.b, cx_e.ik, hv);
                b1.stv(m, ownv(v_xe) | ms, L.oMxe + G(rB) * brow);
            }
            if (!FAST && fy_e(rB)) {
                const float* ct = ctab(rB);
                float m = mfifo[1][fslot(rB)][tid];
                w = cpml_step(m, ct[3], ct[4], ct[5], hv);
                b1.stv(m, v_own | ms, L.oMye + brw(rB) * rowb);
            }
            push(edB, wwB, udB, e, uu, w);
        }
        if (actA) frontA(fast_t, r, fGA[u], fEvA[u], fE[u], fCbA[u], fMxe[u], fMye[u]);
        if (fullB) {                                      // lambda_Hx(hB): own columns
            const float acc = stencil<P>([&](int k) { return wwB[P - 1 + k]; }, [&](int k) { return wwB[P - k]; });
            const float lhx = fmaf(g.rdy, acc, own ? hxA[0] : 0.0f);
            const int mho = M(hx_row(hB) & own_row(hB));
            b1.stv(lhx, v_own | mho, L.oHx + G(hB) * rowb);
            float txv = fQB[u] * lhx;
            if (!FAST && fy_h(hB)) {
                const float* ct = ctab(hB);
                float m = mfifo[2][fslot(hB)][tid];
                txv = cpml_step(m, ct[0], ct[1], ct[2], txv);
                b1.stv(m, v_own | mho, L.oMyh + brw(hB) * rowb);
            }
            shift_in(twB, ((FAST || hx_row(hB)) & own) ? txv : 0.0f);
        }
        if (actA) {                                       // lambda_Hx^n(hA): every E column
            const float acc = stencil<P>([&](int k) { return wwA[P - 1 + k]; }, [&](int k) { return wwA[P - k]; });
            const bool hx_ok = colE & (FAST || hx_row(hA));
            const float lhx = hx_ok ? fmaf(g.rdy, acc, fHx[u]) : 0.0f;
            float txv = fQA[u] * lhx;
            if (!FAST && fy_h(hA)) {
                const float* ct = ctab(hA);
                float m = fMyh[u];
                txv = cpml_step(m, ct[0], ct[1], ct[2], txv);
                mfifo[2][fslot(hA)][tid] = m;
            }
            shift_in(twA, hx_ok ? txv : 0.0f);
            shift_in(hxA, lhx);
        }
        issue(nfast_t, Part1{}, u, rn, live_n);
        rowUB[tid] = udB[0];                              // u of row hB
        rowUA[tid] = udA[0];                              // u of row hA
        __syncthreads();

        // ---- phase 2: lambda_Hz of both stages
        if (fullB && (FAST || hzB_row(hB))) {             // uniform
            const float acc = stencil<P>([&](int k) { return rowUB[th + k]; }, [&](int k) { return rowUB[th - k + 1]; });
            const float lhz = fmaf(-g.rdx, acc, hzA[0]);
            b1.stv(lhz, ownv(v_hzo), L.oHz + (uint32_t)hB * rowb);
            float tz = fQB[u] * lhz;
            if (xband) {
                float m = mfifo[3][fslot(hB)][tid];
                tz = cpml_step(m, cx_h.a, cx_h.b, cx_h.ik, tz);
                b1.stv(m, ownv(v_hzxo), L.oMxh + (uint32_t)hB * brow);
            }
            ringB[rslot(hB % P)][tid] = hzB_ok ? tz : 0.0f;
        }
        if (actA) {
            float hzn = 0.0f;
            if (FAST || hzA_row(hA)) {                    // uniform
                const float acc = stencil<P>([&](int k) { return rowUA[th + k]; }, [&](int k) { return rowUA[th - k + 1]; });
                hzn = hzA_ok ? fmaf(-g.rdx, acc, fHz[u]) : 0.0f;
                float tz = fQA[u] * hzn;
                if (xband) {
                    float m = fMxh[u];
                    tz = cpml_step(m, cx_h.a, cx_h.b, cx_h.ik, tz);
                    mfifo[3][fslot(hA)][tid] = m;
                }
                ringA[rslot((hA + 4 * P) % P)][tid] = hzA_ok ? tz : 0.0f;
            }
            shift_in(hzA, hzn);
        }
        issue(nfast_t, Part2{}, u, rn, live_n);
        __syncthreads();

        // ---- phase 3: lambda_E of both stages
        if (FAST || r >= ya + 4 * P - 1) {                // stage B: yB >= ya (uniform)
            const float* tzr = ringB[yB % P];
            const float az = stencil<P>([&](int k) { return tzr[te + k - 1]; }, [&](int k) { return tzr[te - k]; });
            const float ay = stencil<P>([&](int k) { return twB[P - 1 + k]; }, [&](int k) { return twB[P - k]; });
            b1.stv(fmaf(fCaB[u], edB[0], fmaf(-az, g.rdx, ay * g.rdy)), v_own, L.oE + (uint32_t)yB * rowb);
        }
        if (actA && (FAST || yA >= Ya)) {                 // stage A: lambda_E^n(yA), stage B's next input
            const float* tzr = ringA[(yA + 4 * P) % P];
            const float az = stencil<P>([&](int k) { return tzr[te + k - 1]; }, [&](int k) { return tzr[te - k]; });
            const float ay = stencil<P>([&](int k) { return twA[P - 1 + k]; }, [&](int k) { return twA[P - k]; });
            const float en = fmaf(fCaA[u], edA[0], fmaf(-az, g.rdx, ay * g.rdy));
            eAprev = (eA_ok & (FAST || e_row(yA))) ? en : 0.0f;
        }
        issue(nfast_t, Part3{}, u, rn, live_n);
    };

    // Unrolled blocks starting at r0 in [f_lo, f_hi] without event rows are
    // fast: for every row the block computes and prefetches (r0-4P+1 ..
    // r0+UNROLL-1+D) both stages are active and the rows are owned (stage B),
    // inside the index sets and off the y bands.
    const int f_lo = max(ya, g.y0) + 4 * P - 1;
    constexpr int U = UNROLL_A2;
    const int f_hi = min(min(r_end - 1, g.hy1 - 1), yb + 2 * P - 1) - (U - 1 + D);
    for (int r0 = Ya;; r0 += U) {
        const bool fast = r0 >= f_lo && r0 <= f_hi &&
                          (r0 + U - 1 + D < e_lo || r0 - 2 * P > e_hi);   // uniform
        if (fast) {
#pragma unroll
            for (int uu = 0; uu < U; ++uu) {
                iter(std::true_type{}, std::true_type{}, r0 + uu, uu % D, r0 + uu + D, true);
            }
        } else {
#pragma unroll
            for (int uu = 0; uu < U; ++uu) {
                const int r = r0 + uu;
                if (r > r_end) return;
                iter(std::false_type{}, std::false_type{}, r, uu % D, r + D, r + D <= r_end);
            }
        }
    }
}

}  // namespace tmf
