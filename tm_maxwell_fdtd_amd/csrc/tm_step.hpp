// Fused single-pass time-step kernels of the TM FDTD forward and of its
// exact adjoint (gfx950, wave64).
//
// One launch advances every shot by one time step.  A workgroup of NT = 256
// threads owns a strip of W = NT - 4P + 2 columns and a chunk of CH rows of
// one shot and streams down the chunk one row per iteration:
//   * y-derivatives run on register windows of 2P rows per thread (each
//     thread holds one column);
//   * x-derivatives read a row staged in LDS by the whole workgroup;
//   * the H half-step of a row and the E step of the row P-1 above it are
//     computed in the same iteration, so H never makes a round trip through
//     HBM between the two half-steps.
// Columns within 2P-1 of the strip edges and rows within 2P-1 of the chunk
// edges are read (and their H values recomputed) but written by the
// neighbouring workgroup only.  The state is therefore double-buffered: a
// step reads set 0 and writes set 1 (fields and CPML memories).
//
// Forward step (tide-GPR 0.0.9, maxwell.cu, forward_kernel_h then
// forward_kernel_e):
//   Hx -= Cq filt_y(Dz^h Ey),  Hz += Cq filt_x(Dx^h Ey)          (H rows h)
//   Ey  = Ca Ey + Cb (filt_x(Dx Hz) - filt_y(Dz Hx))             (E rows h-P+1)
// with filt(d) = d / kappa + m, m <- b m + a d inside the CPML bands.
//
// Adjoint step, the exact transpose of the forward step (the same page's
// header comment: time-reversed, transposed operators), per cell:
//   e = lambda_E with the step's residual added at the receivers;
//   gradients (interior); h = Cb e; u, w = band filters of h (own
//   memories, run backwards in time); lambda_Hz -= Dx^h[u];
//   lambda_Hx += Dz^h[w]; t = band filters of Cq lambda_H;
//   lambda_E = Ca e - Dx[t_z] + Dz[t_x].
// The coefficient sits at the source point of each transposed stencil and
// that point's filter comes before the stencil.
//
// Memory access: every load and store is a raw buffer access relative to
// one descriptor per shot and state set (the state of a shot is one
// contiguous block), and lanes that must not touch memory get an offset
// beyond the buffer's range, which reads 0 and drops writes.  The row loop
// is therefore free of per-lane branches; all loads of a row are issued
// PREFETCH rows ahead and, because none is conditional, the in-order
// vector-memory counter lets them stay in flight.  CPML filters along x run
// only in strips that touch an x band (elsewhere the branch is uniform);
// filters along y only on band rows (uniform per row).
//
// Every cell of every output array has exactly one writer; there are no
// atomics.  Floating-point operations are written out explicitly (fmaf
// where a fused multiply-add is wanted) and the library is built without
// contraction, so every template instance computes bitwise the same values
// (a checkpoint replay reproduces the original forward exactly).
#pragma once

#include "tm_common.hpp"

namespace tmf {

constexpr int NT = 256;      // threads per workgroup (4 waves)
constexpr int PREFETCH = 2;  // rows of global loads in flight ahead of the computed row
constexpr int UNROLL = 4;    // row-loop unroll, a multiple of PREFETCH
constexpr int CH_MAX = 256;  // largest chunk height (rows) the LDS tables hold

template <int P>
struct Strip {
    static constexpr int W = NT - 4 * P + 2;   // owned columns per strip
    static constexpr int OFF = 2 * P - 1;      // thread of the first owned column
};

// Launch geometry of the step kernels.
//
// One-step kernels: every strip is cut into nchunk chunks of CH rows.
// Two-step kernels: the nbl leftmost and nbr rightmost strips (those with
// x-band lanes) are cut into nb_ch chunks each, the others into ni_ch, and
// chunk k of n spans the rows between the k/n and (k+1)/n quantiles of a
// row weight (wb outside the rows [wy0, wy1), wi inside), so that the
// slower band rows and band strips get smaller tiles.  Any such cut covers
// every row of every strip exactly once, so the results do not depend on it.
struct Tiling {
    int W, CH;            // owned columns per strip, owned rows per chunk (one-step)
    int nstrip, nchunk;   // strips per row, chunks per column (one-step)
    int nblk;             // workgroups of a launch
    int per_shot;         // two-step: tiles per shot
    int nbl, nbr;         // two-step: band strips at the left / right edge
    int nb_ch, ni_ch;     // two-step: chunks per band strip / per other strip
    int wy0, wy1, wi, wb; // two-step: row weights
};

// Workgroup id -> logical tile id.  Workgroups are dealt round-robin to the
// 8 XCDs; the remap gives each XCD a contiguous range of logical ids, so
// vertically adjacent chunks (which share halo rows) run on the same XCD
// and meet in its L2.
__device__ __forceinline__ int xcd_logical(int nblk)
{
    const int L = blockIdx.x;
    const int q = nblk >> 3, rem = nblk & 7;
    const int xcd = L & 7, j = L >> 3;
    return xcd * q + (xcd < rem ? xcd : rem) + j;
}

// Workgroup id -> (shot, strip, chunk) of the one-step kernels.
__device__ __forceinline__ void tile_of(const Tiling& t, int& s, int& strip, int& chunk)
{
    const int logical = xcd_logical(t.nblk);
    chunk = logical % t.nchunk;
    const int rest = logical / t.nchunk;
    strip = rest % t.nstrip;
    s = rest / t.nstrip;
}

// First row of chunk k of n (two-step tiling): the smallest row y of
// [P, ny - P + 1] whose summed row weight over [P, y) reaches
// ceil(k * total / n); k = 0 gives P and k = n gives ny - P + 1.
__host__ __device__ inline int chunk_row(const Tiling& t, int ny, int P, int k, int n)
{
    const int y_end = ny - P + 1;
    const int64_t A = (int64_t)(t.wy0 - P) * t.wb, M = (int64_t)(t.wy1 - t.wy0) * t.wi;
    const int64_t B = (int64_t)(y_end - t.wy1) * t.wb;
    const int64_t T = ((int64_t)k * (A + M + B) + n - 1) / n;
    if (T <= A) return P + (int)((T + t.wb - 1) / t.wb);
    if (T <= A + M) return t.wy0 + (int)((T - A + t.wi - 1) / t.wi);
    return t.wy1 + (int)((T - A - M + t.wb - 1) / t.wb);
}

// Workgroup id -> (shot, strip, owned rows [ya, yb)) of the two-step kernels.
__device__ __forceinline__ void tile2_of(const Tiling& t, int ny, int P, int& s, int& strip, int& ya, int& yb)
{
    const int logical = xcd_logical(t.nblk);
    s = logical / t.per_shot;
    int k = logical - s * t.per_shot;
    const int nb = t.nbl * t.nb_ch, ni = (t.nstrip - t.nbl - t.nbr) * t.ni_ch;
    int n = t.nb_ch, first = 0;
    if (k >= nb + ni) {
        k -= nb + ni;
        first = t.nstrip - t.nbr;
    } else if (k >= nb) {
        k -= nb;
        n = t.ni_ch;
        first = t.nbl;
    }
    const int q = k / n;
    strip = first + q;
    ya = chunk_row(t, ny, P, k - q * n, n);
    yb = chunk_row(t, ny, P, k - q * n + 1, n);
}

// CPML recursion on one point: memory m <- b m + a d; returns d / kappa + m.
// With a = b = 0 and 1/kappa = 1 it is exactly the identity (m becomes 0).
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

// a, b and 1/kappa of one CPML point.
struct Cpml1 {
    float a, b, ik;
};
__device__ __forceinline__ Cpml1 cpml_at(const float* __restrict__ cp, int L, int row_a, int i)
{
    // rows are ordered a, b, kappa for each of the four grids
    return Cpml1{cp[row_a * L + i], cp[(row_a + 1) * L + i], 1.0f / cp[(row_a + 2) * L + i]};
}

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
}

// Raw buffer view of one block of at most 2 GiB.  A lane whose predicate is
// false gets an offset beyond the buffer's range: its load returns 0 and
// its store is dropped, without a memory access and without a branch.
struct RBuf {
    __amdgpu_buffer_rsrc_t r;
    static constexpr int OOB = (int)0x80000000u;   // >= every buffer size
    __device__ __forceinline__ RBuf(const void* p, uint32_t bytes)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000))
    {
        // one opaque value: the compiler keeps the descriptor in its own
        // aligned register quad instead of sharing equal words between
        // descriptors and copying them together before every access
        asm volatile("" : "+s"(r));
    }
    // byte offset `off` (per lane) within the sub-array at byte `base` (uniform)
    __device__ __forceinline__ float ld(bool ok, uint32_t off, uint32_t base) const
    {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, ok ? (int)off : OOB, (int)base, 0));
    }
    __device__ __forceinline__ void st(bool ok, float v, uint32_t off, uint32_t base) const
    {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, ok ? (int)off : OOB, (int)base, 0);
    }
    // per-lane offset `voff` (already OOB where masked), uniform offset `soff`
    __device__ __forceinline__ float ldv(int voff, uint32_t soff) const
    {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, (int)soff, 0));
    }
    __device__ __forceinline__ void stv(float v, int voff, uint32_t soff) const
    {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, (int)soff, 0);
    }
};

// Lane offset, or the out-of-range offset where the lane is masked.
__device__ __forceinline__ int lane_off(bool ok, uint32_t off) { return ok ? (int)off : RBuf::OOB; }

// Snapshot pairs.  A stored step keeps Ey^n and curl H^n of each interior
// cell side by side ([Ey, curl H] per cell, twice the element size), so one
// access of 2, 4 or 8 bytes moves both values of a cell: [S][nyi][nxi][2]
// per stored step.  Masked lanes (offset out of range) store nothing and
// read (0, 0).
struct SnapPair {
    float e, c;
};
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

template <int SNAP>
constexpr uint32_t pair_bytes() { return 2u * snap_bytes<SNAP>(); }

// Store with a lane offset (bytes, out of range where masked) and a uniform
// row offset.
template <int SNAP>
__device__ __forceinline__ void snap_put2v(const RBuf& b, float e, float c, int voff, uint32_t soff)
{
    if constexpr (SNAP == SNAP_F32) {
        const u32x2_t v = {__float_as_uint(e), __float_as_uint(c)};
        __builtin_amdgcn_raw_buffer_store_b64(v, b.r, voff, (int)soff, 0);
    } else if constexpr (SNAP == SNAP_BF16) {
        const uint32_t v = (uint32_t)f32_to_bf16(e) | ((uint32_t)f32_to_bf16(c) << 16);
        __builtin_amdgcn_raw_buffer_store_b32(v, b.r, voff, (int)soff, 0);
    } else if constexpr (SNAP == SNAP_FP8) {
        const uint32_t v = f32_to_e4m3(e) | (f32_to_e4m3(c) << 8);
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)v, b.r, voff, (int)soff, 0);
    }
}
template <int SNAP>
__device__ __forceinline__ SnapPair snap_get2v(const RBuf& b, int voff, uint32_t soff)
{
    if constexpr (SNAP == SNAP_F32) {
        const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(b.r, voff, (int)soff, 0);
        return SnapPair{__uint_as_float(v.x), __uint_as_float(v.y)};
    } else if constexpr (SNAP == SNAP_BF16) {
        const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(b.r, voff, (int)soff, 0);
        return SnapPair{__uint_as_float(v << 16), __uint_as_float(v & 0xffff0000u)};
    } else if constexpr (SNAP == SNAP_FP8) {
        const uint32_t v = __builtin_amdgcn_raw_buffer_load_b16(b.r, voff, (int)soff, 0);
        return SnapPair{e4m3_to_f32(v & 0xffu), e4m3_to_f32(v >> 8)};
    } else {
        return SnapPair{0.0f, 0.0f};
    }
}
// ... with a predicate and the pair index w of the cell
template <int SNAP>
__device__ __forceinline__ void snap_put2(const RBuf& b, bool ok, uint32_t w, float e, float c)
{
    snap_put2v<SNAP>(b, e, c, lane_off(ok, w * pair_bytes<SNAP>()), 0u);
}
template <int SNAP>
__device__ __forceinline__ SnapPair snap_get2(const RBuf& b, bool ok, uint32_t w)
{
    return snap_get2v<SNAP>(b, lane_off(ok, w * pair_bytes<SNAP>()), 0u);
}

// Layout of one shot's state block (byte offsets of the sub-arrays).
struct StateLayout {
    uint32_t shot_bytes;             // bytes of one shot's block
    uint32_t oE, oHx, oHz;           // fields [ny][nx]
    uint32_t oMyh, oMxh;             // H-update memories: y bands [by][nx], x bands [ny][bx]
    uint32_t oMye, oMxe;             // E-update memories: y bands [by][nx], x bands [ny][bx]
};

// Model block [Ca | Cb | Cq], each [ny][nx]; with one model per shot, shot
// s's block starts shot_stride bytes after shot s-1's (0: one shared block).
struct Model {
    const char* __restrict__ base;
    uint32_t bytes;
    uint32_t oCa, oCb, oCq;
    int64_t shot_stride;
};

// Sources and receivers (tide-GPR 0.0.9, maxwell.cu: add_sources_ey and
// record_receivers_ey, and their adjoints add_adjoint_sources_ey and
// record_adjoint_at_sources).  The grid rows of a shot that hold sources or
// receivers are "event rows", numbered by a slot g (row_slot, -1 for the
// others).  Before a run of steps a small kernel sums each step's inputs
// per cell into dense rows add[g][x] (0 at cells without inputs); a step
// kernel loads the add row of an event row with the field row, adds it to
// the field wherever it computes the row (halo lanes included, so every
// workgroup sees the same values), and the owner of each cell writes the
// field after the addition to out[g][x].  A gather kernel then picks the
// receivers (forward) or the sources (adjoint) out of the out rows.  The
// forward adds sources and reads receivers; the adjoint adds the residual
// at the receivers and reads the sources.
struct EventRows {
    const int* __restrict__ row_slot;   // [S*ny]: slot of (shot, row), or -1
    char* __restrict__ base;            // the event-row buffers of the run (one view)
    uint32_t bytes;                     // of the view
};
// Byte offsets within EventRows::base of one step's add rows and out rows
// [NS][nx] (both always inside the view: a step without inputs adds rows of
// zeros, and out rows nobody gathers are simply not read).
struct EventStep {
    uint32_t add, out;
};

// Slots of rows y_first .. y_first+n-1 of shot s into LDS (-1 outside the
// grid) and the first / last of those rows that are event rows into
// *lo / *hi, which the caller set to INT32_MAX / INT32_MIN before a barrier;
// the caller synchronises afterwards.
__device__ __forceinline__ void load_row_slots(int* t, int* lo, int* hi, const int* __restrict__ row_slot, int s,
                                               int ny, int y_first, int n)
{
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int y = y_first + i;
        const int g = (y >= 0 && y < ny) ? row_slot[s * ny + y] : -1;
        t[i] = g;
        if (g >= 0) {
            atomicMin(lo, y);
            atomicMax(hi, y);
        }
    }
}

// ---------------------------------------------------------------------------
// Forward step
// ---------------------------------------------------------------------------
struct FwdArgs {
    Geo g;
    Tiling t;
    StateLayout L;
    Model m;
    const float* __restrict__ cp;      // CPML table [12][L]
    const char* __restrict__ set0;     // state at step n, shot-major blocks
    char* __restrict__ set1;           // state at step n+1
    char* __restrict__ snap;           // (Ey^n, curl H^n) pairs on the interior window [S][nyi][nxi][2], or null
    uint32_t snap_shot_bytes;          // bytes of one shot's pairs
    EventRows ev;                      // sources (add) and receivers (out)
    EventStep es;                      // ... of this step
};

template <int P, int SNAP>
__global__ __launch_bounds__(NT) void k_fwd_step(FwdArgs a)
{
    constexpr int W = Strip<P>::W, OFF = Strip<P>::OFF;
    constexpr int D = PREFETCH;
    __shared__ float rowE[2][NT];       // by row parity (one barrier per row for P >= 2)
    __shared__ float ring[P][NT];
    __shared__ float cyt[CH_MAX + 2 * P][6];
    __shared__ int evs[CH_MAX];         // slots of the owned rows
    __shared__ int ev_lo, ev_hi;        // first / last owned event row

    const Geo& g = a.g;
    const StateLayout& L = a.L;
    int s, strip, chunk;
    tile_of(a.t, s, strip, chunk);
    const int tid = threadIdx.x;
    const int nx = g.nx, ny = g.ny;
    const int xs = P + strip * W;
    const int xe = min(xs + W, nx - P + 1);
    const int ya = P + chunk * a.t.CH;
    const int yb = min(ya + a.t.CH, ny - P + 1);
    if (tid == 0) {
        ev_lo = INT32_MAX;
        ev_hi = INT32_MIN;
    }
    __syncthreads();
    load_row_cpml(cyt, a.cp, g, ya - P, yb - ya + 2 * P - 1);   // rows ya-P .. yb+P-2
    load_row_slots(evs, &ev_lo, &ev_hi, a.ev.row_slot, s, ny, ya, yb - ya);
    __syncthreads();
    const int e_lo = ev_lo, e_hi = ev_hi;

    const int c = xs - OFF + tid;                       // this thread's column
    const bool own = c >= xs && c < xe;
    const bool incol = c >= 0 && c < nx;
    const bool hz_col = tid >= P - 1 && tid <= NT - P - 1 && c >= P && c <= nx - P - 1;
    const bool fx_h = incol && (c < g.x0 || c >= g.hx1);   // H-update x flag
    const bool fx_e = incol && (c < g.x0 || c >= g.x1);    // E-update x flag
    const bool in_x = c >= g.x0 && c < g.x1;               // interior window column
    const int c0 = xs - OFF;                               // first column of the strip
    const bool xband = c0 < g.x0 || c0 + NT - 1 >= g.hx1;  // uniform: strip touches an x band
    const int bxc = band_x(g, incol ? c : 0);
    const int th = min(max(tid, P - 1), NT - P - 1);       // clamped LDS index for the Hz stencil
    const int te = min(max(tid, P), NT - P);               // ... for the E stencil

    Cpml1 cx_h{0.f, 0.f, 1.f}, cx_e{0.f, 0.f, 1.f};     // identity off the x bands
    if (fx_h) cx_h = cpml_at(a.cp, g.L, AXH, c);
    if (fx_e) cx_e = cpml_at(a.cp, g.L, AX, c);

    auto hx_row = [&](int h) { return h >= P && h <= ny - P - 1; };
    auto h_own = [&](int h) { return h >= ya && h < yb; };
    auto hz_row = [&](int h) { return h_own(h) && h >= P && h <= ny - P; };
    auto fy_h = [&](int h) { return h < g.y0 || h >= g.hy1; };
    auto fy_e = [&](int y) { return y < g.y0 || y >= g.y1; };

    const RBuf b0(a.set0 + (int64_t)s * L.shot_bytes, L.shot_bytes);
    const RBuf b1(a.set1 + (int64_t)s * L.shot_bytes, L.shot_bytes);
    const RBuf bm(a.m.base + (int64_t)s * a.m.shot_stride, a.m.bytes);
    const RBuf bsp(a.snap + (int64_t)s * a.snap_shot_bytes, SNAP != SNAP_NONE ? a.snap_shot_bytes : 0u);
    const RBuf bev(a.ev.base, a.ev.bytes);
    const uint32_t c4 = (uint32_t)c * 4u, bx4 = (uint32_t)bxc * 4u;

    // Prefetch ring: every global load of iteration r is issued at
    // iteration r - D into slot (r - ya) % D; `live` is false past the end
    // of the chunk (those loads are still issued, out of range).
    float fE[D], fQ[D], fHx[D], fHz[D], fCa[D], fCb[D], fMyh[D], fMxh[D], fMxe[D], fMye[D], fEv[D];
    int fG[D];                                          // slot of the E row, or -1 (uniform)
    auto issue = [&](int u, int r, bool live) {
        const int h = r - P, y = r - 2 * P + 1;
        const int gs = (y >= e_lo && y <= e_hi) ? __builtin_amdgcn_readfirstlane(evs[y - ya]) : -1;
        fG[u] = gs;
        fEv[u] = 0.0f;
        if (gs >= 0) fEv[u] = bev.ld(live && own, (uint32_t)(gs * nx) * 4u + c4, a.es.add);   // uniform
        const uint32_t oh = (uint32_t)(h * nx) * 4u + c4, oy = (uint32_t)(y * nx) * 4u + c4;
        fE[u] = b0.ld(live && r >= 0 && r < ny && incol, (uint32_t)(r * nx) * 4u + c4, L.oE);
        fQ[u] = bm.ld(live && incol && (hx_row(h) || h_own(h)), oh, a.m.oCq);
        const bool hx_do = live && own && hx_row(h);
        fHx[u] = b0.ld(hx_do, oh, L.oHx);
        fMyh[u] = b0.ld(hx_do && fy_h(h), (uint32_t)(band_y(g, h) * nx) * 4u + c4, L.oMyh);
        const bool hz_do = live && hz_col && hz_row(h);
        fHz[u] = b0.ld(hz_do, oh, L.oHz);
        fMxh[u] = b0.ld(hz_do && fx_h, (uint32_t)(h * g.bx) * 4u + bx4, L.oMxh);
        const bool e_do = live && own && y >= ya && y < yb;
        fCa[u] = bm.ld(e_do, oy, a.m.oCa);
        fCb[u] = bm.ld(e_do, oy, a.m.oCb);
        fMxe[u] = b0.ld(e_do && fx_e, (uint32_t)(y * g.bx) * 4u + bx4, L.oMxe);
        fMye[u] = b0.ld(e_do && fy_e(y), (uint32_t)(band_y(g, y) * nx) * 4u + c4, L.oMye);
    };

    float ew[2 * P];      // E^n rows r-2P+1 .. r
    float hw[2 * P];      // Hx^{n+1/2} rows r-3P+1 .. r-P
#pragma unroll
    for (int i = 0; i < 2 * P; ++i) { hw[i] = 0.0f; ew[i] = 0.0f; }
#pragma unroll
    for (int i = 1; i < 2 * P; ++i) {
        const int r = ya - 2 * P + i;
        ew[i] = b0.ld(r >= 0 && r < ny && incol, (uint32_t)(r * nx) * 4u + c4, L.oE);
    }
    const int r_end = yb + 2 * P - 2;
#pragma unroll
    for (int u = 0; u < D; ++u) issue(u, ya + u, ya + u <= r_end);

    // The loop ends with the kernel (return, not break), so the latch of the
    // unrolled loop only ever sees a full UNROLL of iterations.
    for (int r0 = ya;; r0 += UNROLL) {
#pragma unroll
        for (int uu = 0; uu < UNROLL; ++uu) {
            const int r = r0 + uu;
            if (r > r_end) return;
            const int u = uu % D;
            const int h = r - P;                       // H row of this iteration
            const int y = r - 2 * P + 1;               // E row of this iteration
            const uint32_t oh = (uint32_t)(h * nx) * 4u + c4;

            // --- rotate the E window
#pragma unroll
            for (int i = 0; i < 2 * P - 1; ++i) ew[i] = ew[i + 1];
            ew[2 * P - 1] = fE[u];

            // --- Hx(h, c): own columns, every H row of the window
            {
                float d = g.rdy * stencil<P>([&](int k) { return ew[P - 1 + k]; },
                                             [&](int k) { return ew[P - k]; });
                const bool st_h = own && hx_row(h) && h_own(h);
                if (fy_h(h)) {                              // uniform
                    const float* ct = cyt[h - ya + P];
                    float m = fMyh[u];
                    d = cpml_step(m, ct[0], ct[1], ct[2], d);
                    b1.st(st_h, m, (uint32_t)(band_y(g, h) * nx) * 4u + c4, L.oMyh);
                }
                const float hxn = (own && hx_row(h)) ? fmaf(-fQ[u], d, fHx[u]) : 0.0f;
                b1.st(st_h, hxn, oh, L.oHx);
#pragma unroll
                for (int i = 0; i < 2 * P - 1; ++i) hw[i] = hw[i + 1];
                hw[2 * P - 1] = hxn;
            }
            float* const rE = rowE[r & 1];
            rE[tid] = ew[P - 1];                       // E^n row h
            __syncthreads();

            // --- Hz(h, c): the owned rows, owned columns plus P on each side
            if (hz_row(h)) {                            // uniform
                float d = g.rdx * stencil<P>([&](int k) { return rE[th + k]; },
                                             [&](int k) { return rE[th - k + 1]; });
                if (xband) {                            // uniform
                    float m = fMxh[u];
                    d = cpml_step(m, cx_h.a, cx_h.b, cx_h.ik, d);
                    b1.st(own && hz_col && fx_h, m, (uint32_t)(h * g.bx) * 4u + bx4, L.oMxh);
                }
                const float hzn = hz_col ? fmaf(fQ[u], d, fHz[u]) : 0.0f;
                b1.st(own && hz_col, hzn, oh, L.oHz);
                ring[h % P][tid] = hzn;
            }
            // P >= 2: the E row reads the ring row written P-1 rows earlier
            // (barriers in between), and the row buffer alternates, so one
            // barrier per row suffices
            if constexpr (P == 1) __syncthreads();

            // --- Ey(y, c): owned cells
            if (y >= ya) {                              // uniform
                const float* hzr = ring[y % P];
                float uu_ = g.rdx * stencil<P>([&](int k) { return hzr[te + k - 1]; },
                                               [&](int k) { return hzr[te - k]; });
                if (xband) {
                    float m = fMxe[u];
                    uu_ = cpml_step(m, cx_e.a, cx_e.b, cx_e.ik, uu_);
                    b1.st(own && fx_e, m, (uint32_t)(y * g.bx) * 4u + bx4, L.oMxe);
                }
                float v = g.rdy * stencil<P>([&](int k) { return hw[P - 1 + k]; },
                                             [&](int k) { return hw[P - k]; });
                if (fy_e(y)) {
                    const float* ct = cyt[y - ya + P];
                    float m = fMye[u];
                    v = cpml_step(m, ct[3], ct[4], ct[5], v);
                    b1.st(own, m, (uint32_t)(band_y(g, y) * nx) * 4u + c4, L.oMye);
                }
                const float curl = uu_ - v;
                const float ev = ew[0];
                if constexpr (SNAP != SNAP_NONE) {
                    if (y >= g.y0 && y < g.y1) {
                        const uint32_t w = (uint32_t)((y - g.y0) * g.nxi + (c - g.x0));
                        snap_put2<SNAP>(bsp, own && in_x, w, ev, curl);
                    }
                }
                float en = fmaf(fCa[u], ev, fCb[u] * curl);
                if (fG[u] >= 0) {                       // uniform: sources, then receivers
                    en = en + fEv[u];
                    bev.st(own, en, (uint32_t)(fG[u] * nx) * 4u + c4, a.es.out);
                }
                b1.st(own, en, (uint32_t)(y * nx) * 4u + c4, L.oE);
            }
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
    StateLayout L;     // oMyh / oMxh: adjoint memories of the Hx / Hz filters;
                       // oMye / oMxe: of the E-update y / x filters
    Model m;
    const float* __restrict__ cp;
    const char* __restrict__ set0;     // adjoint state after step n+1
    char* __restrict__ set1;           // adjoint state after step n
    const char* __restrict__ snap;     // (Ey^n, curl H^n) pairs of this step [S][nyi][nxi][2], or null
    uint32_t snap_shot_bytes;          // bytes of one shot's pairs
    float* __restrict__ gca;           // per-shot gradients [S][ny][nx], or null
    float* __restrict__ gcb;
    float ratio;                       // weight of this step's gradient term (the snapshot step ratio)
    EventRows ev;                      // residual at the receivers (add), sources (out)
    EventStep es;                      // ... of this step
};

template <int P, int SNAP>
__global__ __launch_bounds__(NT) void k_adj_step(AdjArgs a)
{
    constexpr int W = Strip<P>::W, OFF = Strip<P>::OFF;
    constexpr int D = PREFETCH;
    constexpr int T0 = 2 * P - 1;      // LDS table index of row y is y - ya + T0
    __shared__ float rowU[NT];
    __shared__ float ring[P][NT];
    __shared__ float cyt[CH_MAX + 4 * P][6];
    __shared__ int evs[CH_MAX + 4 * P];         // row slots, indexed like cyt
    __shared__ int ev_lo, ev_hi;                // first / last event row of the window

    const Geo& g = a.g;
    const StateLayout& L = a.L;
    int s, strip, chunk;
    tile_of(a.t, s, strip, chunk);
    const int tid = threadIdx.x;
    const int nx = g.nx, ny = g.ny;
    const int xs = P + strip * W;
    const int xe = min(xs + W, nx - P + 1);
    const int ya = P + chunk * a.t.CH;
    const int yb = min(ya + a.t.CH, ny - P + 1);
    if (tid == 0) {
        ev_lo = INT32_MAX;
        ev_hi = INT32_MIN;
    }
    __syncthreads();
    load_row_cpml(cyt, a.cp, g, ya - T0, yb - ya + 4 * P - 2);   // rows ya-2P+1 .. yb+2P-2
    load_row_slots(evs, &ev_lo, &ev_hi, a.ev.row_slot, s, ny, ya - T0, yb - ya + 4 * P - 2);
    __syncthreads();
    const int e_lo = ev_lo, e_hi = ev_hi;

    const int c = xs - OFF + tid;
    const bool own = c >= xs && c < xe;
    const bool e_col = c >= P && c <= nx - P;          // E-set column
    const bool hz_col = tid >= P - 1 && tid <= NT - P - 1 && c >= P && c <= nx - P - 1;
    const bool fx_h = e_col && (c < g.x0 || c >= g.hx1);
    const bool fx_e = e_col && (c < g.x0 || c >= g.x1);
    const bool in_x = c >= g.x0 && c < g.x1;
    const int c0 = xs - OFF;
    const bool xband = c0 < g.x0 || c0 + NT - 1 >= g.hx1;
    const int bxc = band_x(g, (c >= 0 && c < nx) ? c : 0);
    const int th = min(max(tid, P - 1), NT - P - 1);
    const int te = min(max(tid, P), NT - P);
    const bool grad = SNAP != SNAP_NONE && own && in_x;

    Cpml1 cx_h{0.f, 0.f, 1.f}, cx_e{0.f, 0.f, 1.f};
    if (fx_h) cx_h = cpml_at(a.cp, g.L, AXH, c);
    if (fx_e) cx_e = cpml_at(a.cp, g.L, AX, c);

    auto hx_row = [&](int h) { return h >= P && h <= ny - P - 1; };
    auto h_own = [&](int h) { return h >= ya && h < yb; };
    auto hz_row = [&](int h) { return h_own(h) && h >= P && h <= ny - P; };
    auto e_row = [&](int r) { return r >= P && r <= ny - P; };
    auto fy_h = [&](int h) { return h < g.y0 || h >= g.hy1; };
    auto fy_e = [&](int y) { return y < g.y0 || y >= g.y1; };

    const RBuf b0(a.set0 + (int64_t)s * L.shot_bytes, L.shot_bytes);
    const RBuf b1(a.set1 + (int64_t)s * L.shot_bytes, L.shot_bytes);
    const RBuf bm(a.m.base + (int64_t)s * a.m.shot_stride, a.m.bytes);
    constexpr uint32_t ESZ = snap_bytes<SNAP>();
    const uint32_t ssb = SNAP != SNAP_NONE ? a.snap_shot_bytes : 0u;
    const RBuf bsp(a.snap + (int64_t)s * a.snap_shot_bytes, ssb);
    const uint32_t slab_b = (uint32_t)(g.slab * 4);
    const RBuf bga(a.gca + (int64_t)s * g.slab, a.gca ? slab_b : 0u);
    const RBuf bgb(a.gcb + (int64_t)s * g.slab, a.gcb ? slab_b : 0u);
    const RBuf bev(a.ev.base, a.ev.bytes);
    const uint32_t c4 = (uint32_t)c * 4u, bx4 = (uint32_t)bxc * 4u;
    const uint32_t rowb = (uint32_t)nx * 4u, brow = (uint32_t)g.bx * 4u;

    // Addressing: the lane part of an offset is loop-invariant and already
    // out of range where the lane never touches that array; a row's
    // conditions OR in a uniform mask (0, or out of range); the row part is
    // a uniform offset of the row clamped into the array, so that a masked
    // offset plus the row offset never wraps back into range.
    const int v_e = lane_off(e_col, c4), v_own = lane_off(own, c4);
    const int v_hz = lane_off(hz_col, c4), v_ownhz = lane_off(own && hz_col, c4);
    const int v_xe = lane_off(fx_e, bx4), v_ownxe = lane_off(own && fx_e, bx4);
    const int v_hzxh = lane_off(hz_col && fx_h, bx4), v_ownhzxh = lane_off(own && hz_col && fx_h, bx4);
    const int v_g = lane_off(grad, c4), v_gs = lane_off(grad, (uint32_t)(c - g.x0) * 2u * ESZ);
    auto msk = [](bool ok) { return ok ? 0 : RBuf::OOB; };
    auto grow = [&](int y) { return (uint32_t)min(max(y, 0), ny - 1); };                // grid row
    auto brw = [&](int y) { return (uint32_t)min(max(band_y(g, y), 0), g.by - 1); };    // y-band row
    auto srw = [&](int y) { return (uint32_t)min(max(y - g.y0, 0), g.nyi - 1) * (uint32_t)g.nxi * 2u * ESZ; };
    // slot of window row r, or -1 (uniform)
    auto slot_of = [&](int r) {
        return (r >= e_lo && r <= e_hi) ? __builtin_amdgcn_readfirstlane(evs[r - ya + T0]) : -1;
    };

    // Prefetch ring (see k_fwd_step).
    float fE[D], fCb[D], fMxe[D], fMye[D], fSe[D], fSc[D], fGa[D], fGb[D];
    float fHx[D], fMyh[D], fQ[D], fHz[D], fMxh[D], fCa[D], fEv[D];
    int fG[D];
    auto issue = [&](int u, int r, bool live) {
        const int h = r - P, y = r - 2 * P + 1;
        const int me = msk(live && e_row(r));
        const uint32_t orr = grow(r) * rowb, oh = grow(h) * rowb;
        const int gs = slot_of(r);
        fG[u] = gs;
        fEv[u] = 0.0f;
        if (gs >= 0) fEv[u] = bev.ldv(v_e | me, (uint32_t)gs * rowb + a.es.add);   // uniform
        fE[u] = b0.ldv(v_e | me, L.oE + orr);
        fCb[u] = bm.ldv(v_e | me, a.m.oCb + orr);
        fMxe[u] = b0.ldv(v_xe | me, L.oMxe + grow(r) * brow);
        fMye[u] = b0.ldv(v_e | me | msk(fy_e(r)), L.oMye + brw(r) * rowb);
        const int mg = msk(live && r >= ya && r < yb && r >= g.y0 && r < g.y1);
        const SnapPair sp = snap_get2v<SNAP>(bsp, v_gs | mg, srw(r));
        fSe[u] = sp.e;
        fSc[u] = sp.c;
        fGa[u] = bga.ldv(v_g | mg, orr);
        fGb[u] = bgb.ldv(v_g | mg, orr);
        const int mh = msk(live && hx_row(h));
        fHx[u] = b0.ldv(v_own | mh, L.oHx + oh);
        fMyh[u] = b0.ldv(v_own | mh | msk(fy_h(h)), L.oMyh + brw(h) * rowb);
        fQ[u] = bm.ldv(v_e | msk(live && (hx_row(h) || h_own(h))), a.m.oCq + oh);
        const int mz = msk(live && hz_row(h));
        fHz[u] = b0.ldv(v_hz | mz, L.oHz + oh);
        fMxh[u] = b0.ldv(v_hzxh | mz, L.oMxh + grow(h) * brow);
        fCa[u] = bm.ldv(v_own | msk(live && y >= ya && y < yb), a.m.oCa + grow(y) * rowb);
    };

    float ed[2 * P];      // lambda_E^{n+1} rows r-2P+1 .. r
    float ww[2 * P];      // filtered Cb lambda_E for the Hx transpose, rows r-2P+1 .. r
    float ud[P + 1];      // filtered Cb lambda_E for the Hz transpose, rows r-P .. r
    float tw[2 * P];      // filtered Cq lambda_Hx, rows r-3P+1 .. r-P
#pragma unroll
    for (int i = 0; i < 2 * P; ++i) { ed[i] = 0.0f; ww[i] = 0.0f; tw[i] = 0.0f; }
#pragma unroll
    for (int i = 0; i <= P; ++i) ud[i] = 0.0f;

    // lambda_E^{n+1} of row r (slot gs, add-row value ev) with the step's
    // residual added at the receivers: every workgroup reading the row adds
    // it; the owner of the cell keeps the result (source-wavelet gradient).
    auto inject = [&](int r, int gs, float ev, float e) {
        if (gs >= 0) {                                  // uniform
            e = e + ev;
            bev.stv(e, v_own | msk(r >= ya && r < yb), (uint32_t)gs * rowb + a.es.out);
        }
        return e;
    };
    // u, w of the E-set cell (r, c) for input row r (0 off the E-set); the
    // filter memories are written back on owned cells.
    auto front = [&](int r, float e, float cbv, float mx, float my, float& u, float& w) {
        const int ms = msk(r >= ya && r < yb && e_row(r));    // owned E-set rows
        const float hv = cbv * e;
        u = hv;
        if (xband) {
            float m = mx;
            u = cpml_step(m, cx_e.a, cx_e.b, cx_e.ik, hv);
            b1.stv(m, v_ownxe | ms, L.oMxe + grow(r) * brow);
        }
        w = hv;
        if (fy_e(r)) {
            const float* ct = cyt[r - ya + T0];
            float m = my;
            w = cpml_step(m, ct[3], ct[4], ct[5], hv);
            b1.stv(m, v_own | ms, L.oMye + brw(r) * rowb);
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
    for (int i = 1; i < 2 * P; ++i) {
        const int r = ya - 2 * P + i;
        const int me = msk(e_row(r));
        const uint32_t orr = grow(r) * rowb;
        const int gs = slot_of(r);
        float ev = 0.0f;
        if (gs >= 0) ev = bev.ldv(v_e | me, (uint32_t)gs * rowb + a.es.add);   // uniform
        const float e0 = inject(r, gs, ev, b0.ldv(v_e | me, L.oE + orr)), cbv = bm.ldv(v_e | me, a.m.oCb + orr);
        const float mx = b0.ldv(v_xe | me, L.oMxe + grow(r) * brow);
        const float my = b0.ldv(v_e | me | msk(fy_e(r)), L.oMye + brw(r) * rowb);
        float u, w;
        front(r, e0, cbv, mx, my, u, w);
        push(e0, u, w);
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
                const float e = inject(r, fG[u], fEv[u], fE[u]);
                float uv, wv;
                front(r, e, fCb[u], fMxe[u], fMye[u], uv, wv);
                if constexpr (SNAP != SNAP_NONE) {
                    if (r < yb && r >= g.y0 && r < g.y1) {  // uniform
                        const uint32_t orr = (uint32_t)r * rowb;
                        bga.stv(fmaf(e, fSe[u] * a.ratio, fGa[u]), v_g, orr);
                        bgb.stv(fmaf(e, fSc[u] * a.ratio, fGb[u]), v_g, orr);
                    }
                }
                push(e, uv, wv);
            }
            const int h = r - P;
            const int y = r - 2 * P + 1;
            const float q = fQ[u];

            // --- lambda_Hx(h, c) and its filtered Cq product, own columns
            {
                const bool do_h = own && hx_row(h);
                const float acc = stencil<P>([&](int k) { return ww[P - 1 + k]; },
                                             [&](int k) { return ww[P - k]; });
                const float lhx = fmaf(g.rdy, acc, fHx[u]);
                const int mho = msk(hx_row(h) && h_own(h));
                b1.stv(lhx, v_own | mho, L.oHx + grow(h) * rowb);
                float txv = q * lhx;
                if (fy_h(h)) {                          // uniform
                    const float* ct = cyt[h - ya + T0];
                    float m = fMyh[u];
                    txv = cpml_step(m, ct[0], ct[1], ct[2], txv);
                    b1.stv(m, v_own | mho, L.oMyh + brw(h) * rowb);
                }
#pragma unroll
                for (int i = 0; i < 2 * P - 1; ++i) tw[i] = tw[i + 1];
                tw[2 * P - 1] = do_h ? txv : 0.0f;
            }
            rowU[tid] = ud[0];                          // u of row h
            __syncthreads();

            // --- lambda_Hz(h, c): owned rows, owned columns plus P on each side
            if (hz_row(h)) {                            // uniform
                const float acc = stencil<P>([&](int k) { return rowU[th + k]; },
                                             [&](int k) { return rowU[th - k + 1]; });
                const float lhz = fmaf(-g.rdx, acc, fHz[u]);
                b1.stv(lhz, v_ownhz, L.oHz + (uint32_t)h * rowb);
                float tz = q * lhz;
                if (xband) {
                    float m = fMxh[u];
                    tz = cpml_step(m, cx_h.a, cx_h.b, cx_h.ik, tz);
                    b1.stv(m, v_ownhzxh, L.oMxh + (uint32_t)h * brow);
                }
                ring[h % P][tid] = hz_col ? tz : 0.0f;
            }
            __syncthreads();

            // --- lambda_E(y, c) = Ca e - Dx[t_z] + Dz[t_x]
            if (y >= ya) {                              // uniform
                const float* tzr = ring[y % P];
                const float az = stencil<P>([&](int k) { return tzr[te + k - 1]; },
                                            [&](int k) { return tzr[te - k]; });
                const float ay = stencil<P>([&](int k) { return tw[P - 1 + k]; },
                                            [&](int k) { return tw[P - k]; });
                b1.stv(fmaf(fCa[u], ed[0], fmaf(-az, g.rdx, ay * g.rdy)), v_own, L.oE + (uint32_t)y * rowb);
            }
            issue(u, r + D, r + D <= r_end);
        }
    }
}

}  // namespace tmf
