// Host runtime and C ABI of the TM FDTD propagator (see include/tm_fdtd.h).
//
// The plan validates a problem on the host, builds the per-row event-cell
// tables of the sources and receivers, chooses the tiling of the step kernels and lays
// out the caller-allocated workspace.  tm_forward / tm_adjoint / tm_grad
// enqueue kernels on the caller's stream; there is no global state, so plans
// are independent.
//
// Host loop structure follows the launchers of tide-GPR 0.0.9, maxwell.cu
// (forward, forward_with_storage, backward), with each step's small kernels
// fused into its stencil kernel: per forward step (or pair of steps) one
// kernel (H and E updates, sources, then receivers, snapshot epilogue on
// stored steps); per adjoint step, in reverse time, one kernel (residual
// injection at the receivers, adjoint read at the sources, transposed H and
// E updates, gradient accumulation); then combine_grad.  Checkpoint mode
// stores the state (fields and band CPML memories) every K steps and replays
// each segment into a K-step snapshot buffer inside tm_adjoint.
//
// Workspace: each step reads one state set and writes the other (double
// buffering); a set holds, shot after shot, one contiguous block of fields
// and CPML memories per shot, so a kernel addresses a shot's whole state
// through one buffer descriptor.  The model arrays are copied into one
// block [Ca | Cb | Cq] at the start of each call.  A checkpoint is a copy
// of one set and is restored into set 0.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <utility>
#include <vector>

#include "tm_fdtd.h"
#include "tm_kernels.hpp"
#include "tm_step.hpp"
#include "tm_step2.hpp"
#include "tm_adj2.hpp"
#include "tm_small.hpp"
#include "tm_band.hpp"

using namespace tmf;

#define TM_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr uint64_t ALIGN = 256;
uint64_t align_up(uint64_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }
constexpr uint64_t BLOCK_MAX = (uint64_t(1) << 31) - ALIGN;   // one buffer view
constexpr uint64_t EV_BLOCK_BYTES = uint64_t(16) << 20;        // one event-row buffer (a run of steps)
constexpr uint64_t EV_ROW_MAX = uint64_t(1) << 29;              // one step's event rows (add + out in one view)
constexpr uint64_t SCRATCH_BYTES = 4096;                        // the workspace's scratch area

double abs_coef_sum(int order)
{
    switch (order) {
    case 2: return 1.0;
    case 4: return 9.0 / 8.0 + 1.0 / 24.0;
    case 8: return 1225.0 / 1024.0 + 245.0 / 3072.0 + 49.0 / 5120.0 + 5.0 / 7168.0;
    default: return 0.0;
    }
}

// Event-row tables of the sources and receivers (EventRows): per shot the
// grid rows holding sources or receivers (negative indices = absent) get
// slots g, ascending by shot then row; the distinct cells of those rows are
// numbered k, each with its source indices and its receiver indices
// (ascending, CSR); colcell[g][x] = k or -1; src_pos / rec_pos [S][n] =
// g*nx + x of each entry's cell, or -1.
struct EventTables {
    std::vector<int32_t> row_slot, colcell, slot_shot, cell_src, src_list, cell_rec, rec_list, src_pos, rec_pos;
    int64_t n_slots = 0;
};

EventTables build_events(const int64_t* src, int64_t n_src, const int64_t* rec, int64_t n_rec, int64_t S,
                         int64_t ny, int64_t nx)
{
    EventTables t;
    t.row_slot.assign(S * ny, -1);
    t.src_pos.assign(S * n_src, -1);
    t.rec_pos.assign(S * n_rec, -1);
    std::vector<std::pair<int64_t, int32_t>> v;       // (cell, entry), receivers as entry >= n_src
    for (int64_t s = 0; s < S; ++s) {
        v.clear();
        for (int64_t i = 0; i < n_src; ++i)
            if (src[s * n_src + i] >= 0) v.emplace_back(src[s * n_src + i], (int32_t)i);
        for (int64_t j = 0; j < n_rec; ++j)
            if (rec[s * n_rec + j] >= 0) v.emplace_back(rec[s * n_rec + j], (int32_t)(n_src + j));
        std::sort(v.begin(), v.end());
        for (size_t k = 0; k < v.size(); ++k) {
            const int64_t y = v[k].first / nx, x = v[k].first % nx;
            int32_t& g = t.row_slot[s * ny + y];
            if (g < 0) {                                  // a new event row of this shot
                g = (int32_t)t.n_slots++;
                t.slot_shot.push_back((int32_t)s);
                t.colcell.resize(t.n_slots * nx, -1);
            }
            if (k == 0 || v[k].first != v[k - 1].first) {
                t.colcell[g * nx + x] = (int32_t)t.cell_src.size();
                t.cell_src.push_back((int32_t)t.src_list.size());
                t.cell_rec.push_back((int32_t)t.rec_list.size());
            }
            const int32_t pos = (int32_t)(g * nx + x);
            if (v[k].second < n_src) {
                t.src_list.push_back(v[k].second);
                t.src_pos[s * n_src + v[k].second] = pos;
            } else {
                t.rec_list.push_back((int32_t)(v[k].second - n_src));
                t.rec_pos[s * n_rec + (v[k].second - n_src)] = pos;
            }
        }
    }
    t.cell_src.push_back((int32_t)t.src_list.size());
    t.cell_rec.push_back((int32_t)t.rec_list.size());
    return t;
}

struct Layout {
    uint64_t cpml = 0, tables = 0, scratch = 0;
    uint64_t model = 0, model_bytes = 0;          // [Ca | Cb | Cq] of one model
    uint64_t model_stride = 0;                    // bytes between the shots' models (0: shared)
    uint64_t slab_b = 0;                          // bytes of one [ny][nx] array, aligned
    StateLayout st{};                             // one shot's block (forward and adjoint alike)
    uint64_t set_bytes = 0;                       // S blocks
    uint64_t fwd = 0, fwd_bytes = 0, fset[2] = {0, 0};
    uint64_t adj = 0, adj_bytes = 0, aset[2] = {0, 0};
    uint64_t snap = 0;                            // stored steps: (Ey, curl H) pairs [S][nyi][nxi][2] each
    uint64_t snap_stride = 0;                     // bytes per stored step (all shots)
    uint64_t snap_shot = 0;                       // ... of one shot
    uint64_t ckpt = 0, ckpt_slot = 0;
    uint64_t ev_row = 0;                          // bytes of one step's event rows [NS][nx]
    uint64_t ev_fadd = 0, ev_fout = 0, ev_aadd = 0, ev_aout = 0;   // [EB][NS][nx] each
    uint64_t band_x = 0, band_x_bytes = 0, band_err = 0;   // banded kernels: exchange rows, failure word
    uint64_t total = 0;
};

}  // namespace

// Device slots of the host snapshot store (copies of one slot overlap the
// kernels writing or reading the others).
constexpr int HOST_RING = 3;

// Timed stencil kernels (tm_timing_*): ids and symbol-name prefixes; the
// forward launches that store snapshots are timed apart from the others
// ("_store"), since they move more bytes.
enum KernelId {
    KID_FWD_STEP = 0, KID_ADJ_STEP, KID_FWD_STEP2, KID_ADJ_STEP2, KID_FWD_STEP2_UQ, KID_ADJ_STEP2_UQ,
    KID_FWD_STEP_ST, KID_FWD_STEP2_ST, KID_FWD_STEP2_UQ_ST, KID_FWD_SMALL, KID_FWD_SMALL_ST, KID_ADJ_SMALL,
    KID_FWD_BAND, KID_FWD_BAND_ST, KID_ADJ_BAND, KID_FWD_BANDK, KID_FWD_BANDK_ST, KID_ADJ_BANDK, KID_COUNT
};
const char* const KERNEL_NAMES[KID_COUNT] = {"k_fwd_step", "k_adj_step", "k_fwd_step2", "k_adj_step2",
                                             "k_fwd_step2_uq", "k_adj_step2_uq", "k_fwd_step_store",
                                             "k_fwd_step2_store", "k_fwd_step2_uq_store", "k_fwd_small",
                                             "k_fwd_small_store", "k_adj_small", "k_fwd_band",
                                             "k_fwd_band_store", "k_adj_band", "k_fwd_bandk",
                                             "k_fwd_bandk_store", "k_adj_bandk"};

struct TimedLaunch {
    int kid;
    hipEvent_t a, b;
};

struct tm_plan {
    tm_desc d{};
    int P = 0;
    Geo g{};
    Tiling tiling_fwd{}, tiling_adj{};   // per device, made at the first device call
    Tiling tiling_fwd2{}, tiling_adj2{};
    int time_block = 2;                  // time steps per launch of the streaming kernels (1 or 2)
    int resident = 0;                    // resident kernels: 0 never, 1 where they fit and the shots are
                                         // many (time_block 0), 2 wherever they fit (time_block 3)
    bool small = false;                  // the resident kernels run (per device, with the tilings)
    int band = 0;                        // banded resident kernels: 0 never, 1 for small problems with
                                         // few shots (time_block 0), 2 wherever they fit (time_block 4)
    int band_rb = 0, band_n = 0;         // their band height and bands per shot (0: the grid does not fit)
    int band_kx = 0, band_hd = 0;        // blocked banded kernels: steps per exchange and extended rows
                                         // per side (0: the kernels exchanging twice per step)
    bool banded = false;                 // the banded kernels run (per device)
    bool band_ran = false;               // a banded launch ran in the current call (its failure word is read)
    int tiling_device = -1;
    std::vector<float> cpml;             // [12][L]
    std::vector<int32_t> tables;         // event-row tables, packed
    uint64_t t_slot = 0, t_colcell = 0, t_sshot = 0, t_cs = 0, t_sl = 0, t_cr = 0, t_rl = 0;
    uint64_t t_spos = 0, t_rpos = 0;
    int64_t NS = 0;                      // event rows (all shots)
    int64_t EB = 1;                      // steps per event block
    Layout lay;
    int64_t K = 0, n_seg = 0, n_ckpt = 0, seg_steps = 0;
    // snapshot storage: every R-th step (R = step ratio), on the device or in
    // a pinned host store reached through a ring of device slots
    int64_t R = 1, n_store = 0;
    int storage = TM_STORE_DEVICE;
    char* host_store = nullptr;          // pinned [n_store][S][nyi][nxi][2] (Ey, curl H pairs)
    uint64_t host_bytes = 0;
    hipStream_t copy_stream = nullptr;
    hipEvent_t slot_copied[HOST_RING] = {};   // last copy into / out of the slot finished
    hipEvent_t slot_done[HOST_RING] = {};     // last kernel reading / writing the slot finished
    bool slot_copy_pending[HOST_RING] = {};
    bool slot_kernel_pending[HOST_RING] = {};
    // pinned staging copy of cpml + tables (allocated on first device call)
    void* pinned = nullptr;
    uint64_t pinned_bytes = 0;
    float* readback = nullptr;           // pinned words the host reads back (Courant scan, failure word)
    hipEvent_t readback_done = nullptr;  // ... recorded after their copy
    // sequence state
    void* ws_last = nullptr;
    int64_t fwd_next = -1;
    int fwd_cur = 0;                     // forward set holding the state at fwd_next
    bool stored_ok = false;
    bool fwd_complete = false;
    // during a tm_forward call whose Courant check found Cq to hold one
    // value: that value, read by the two-step forward instead of the array
    bool cq_uniform = false;
    float cq_value = 0.0f;
    // order 8: every strip's x-band lanes fit the compact FIFOs of the
    // two-step forward (then its four-workgroup instances run)
    bool fwd_cx = false;
    // what the checks of the storing forward found: every chunk's Cq held
    // the one value fwd_cq_val, at the pointer fwd_cq (the replays of the
    // adjoint, which take the same arrays, then read no Cq either)
    const float* fwd_cq = nullptr;
    bool fwd_cq_one = false;
    float fwd_cq_val = 0.0f;
    // sampled kernel timing
    int timing_every = 0;
    std::vector<hipEvent_t> ev_free;
    std::vector<TimedLaunch> ev_used;
    double t_ms[KID_COUNT] = {};
    int64_t t_n[KID_COUNT] = {};
};

namespace {

tm_status validate_indices(const int64_t* ids, int64_t S, int64_t n, int64_t ny, int64_t nx, int P)
{
    if (n > 0 && ids == nullptr) return TM_EINVAL;
    for (int64_t k = 0; k < S * n; ++k) {
        const int64_t c = ids[k];
        if (c < 0) continue;
        if (c >= ny * nx) return TM_EINVAL;
        const int64_t y = c / nx, x = c % nx;
        if (y < P || y > ny - P || x < P || x > nx - P) return TM_EINVAL;
    }
    return TM_OK;
}

bool finite_all(const float* p, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        if (!std::isfinite(p[i])) return false;
    return true;
}

// Steps between exchanges of the blocked banded kernels (measured on the
// order-2 86^2 grid with one shot, forward + adjoint: 3 steps 2.32 Gcell/s,
// 2 steps 2.23, 4 steps 2.11); where the extended rows of 3 steps do not
// fit a band, 2.
constexpr int BANDK_STEPS = 3;

// Band height and bands per shot of the banded resident kernels (0: they
// do not apply): as many bands as one workgroup per CU of the device allows
// (256 CUs; the device check repeats it with the real count).  Blocked
// kernels (kx > 0 steps between exchanges, else fewer down to 2): every band but the last owns
// at least hd = kx (2P - 1) rows, and the extended rows fit the packed cell
// word, the threads and the LDS of a CU; where they do not, the kernels
// exchanging every step, with bands of at least max(2P, 4) rows, the last of
// at least P, within the packed cell word and the LDS of a CU.
void band_plan(tm_plan* p, int kx)
{
    p->band_rb = p->band_n = p->band_kx = p->band_hd = 0;
    if (p->band == 0) return;
    const Geo& g = p->g;
    const int64_t S = p->d.n_shots;
    constexpr int64_t WG_MAX = 256;
    if (S > WG_MAX || g.ny >= 2048) return;
    // blocked: every band but the last owns at least hd rows; kx steps
    // between exchanges, else fewer, down to 2
    for (int k = kx; k > 0 && k >= std::min(kx, 2); --k) {
        const int hd = k * (2 * g.P - 1);
        for (int64_t nb = std::min<int64_t>(WG_MAX / S, (g.ny + hd - 1) / hd); nb >= 2; --nb) {
            const int rb = (int)((g.ny + nb - 1) / nb);
            const int n = (g.ny + rb - 1) / rb;
            if (!bandk_rows_ok(g, rb, hd) || bandk_lds_bytes(g, rb, hd, true) > 160u * 1024u) continue;
            p->band_rb = rb;
            p->band_n = n;
            p->band_kx = k;
            p->band_hd = hd;
            return;
        }
    }
    const int rb_min = std::max(2 * g.P, 4);
    for (int64_t nb = std::min<int64_t>(WG_MAX / S, g.ny / rb_min); nb >= 2; --nb) {
        const int rb = (int)((g.ny + nb - 1) / nb);
        const int n = (g.ny + rb - 1) / rb;
        if (g.ny - (n - 1) * rb < g.P || !band_rows_ok(g, rb)) continue;
        if (band_lds_bytes(g, rb, true) > 160u * 1024u) continue;
        p->band_rb = rb;
        p->band_n = n;
        return;
    }
}

// Returns false when a per-shot block or the model block exceeds one
// buffer view.
bool make_layout(tm_plan* p)
{
    const tm_desc& d = p->d;
    const Geo& g = p->g;
    Layout& L = p->lay;
    const uint64_t S = (uint64_t)d.n_shots;
    L.slab_b = align_up((uint64_t)g.slab * 4);
    const uint64_t yb = align_up((uint64_t)g.by * (uint64_t)g.nx * 4);
    const uint64_t xb = align_up((uint64_t)g.ny * (uint64_t)g.bx * 4);
    const uint64_t shot = 3 * L.slab_b + 2 * yb + 2 * xb;
    if (shot > BLOCK_MAX || 3 * L.slab_b > BLOCK_MAX) return false;
    L.st.shot_bytes = (uint32_t)shot;
    L.st.oE = 0;
    L.st.oHx = (uint32_t)L.slab_b;
    L.st.oHz = (uint32_t)(2 * L.slab_b);
    L.st.oMyh = (uint32_t)(3 * L.slab_b);
    L.st.oMxh = (uint32_t)(3 * L.slab_b + yb);
    L.st.oMye = (uint32_t)(3 * L.slab_b + yb + xb);
    L.st.oMxe = (uint32_t)(3 * L.slab_b + 2 * yb + xb);
    L.set_bytes = S * shot;

    uint64_t o = 0;
    auto take = [&](uint64_t bytes) { uint64_t at = o; o = align_up(o + bytes); return at; };
    L.cpml = take(12 * (uint64_t)g.L * 4);
    L.tables = take(p->tables.size() * 4);
    L.scratch = take(SCRATCH_BYTES);
    L.model_bytes = 3 * L.slab_b;
    L.model_stride = d.model_per_shot ? L.model_bytes : 0;
    L.model = take(L.model_bytes * (d.model_per_shot ? S : 1));
    L.fwd = o;
    L.fset[0] = take(L.set_bytes);
    L.fset[1] = take(L.set_bytes);
    L.fwd_bytes = o - L.fwd;
    L.adj = o;
    L.aset[0] = take(L.set_bytes);
    L.aset[1] = take(L.set_bytes);
    L.adj_bytes = o - L.adj;
    const uint64_t esz = d.snap == TM_SNAP_BF16 ? 2 : d.snap == TM_SNAP_FP8 ? 1 : 4;
    L.snap_shot = (uint64_t)g.nyi * (uint64_t)g.nxi * 2 * esz;
    const uint64_t dev_steps = p->storage == TM_STORE_HOST ? (uint64_t)HOST_RING
                             : p->K > 0 ? (uint64_t)p->seg_steps : (uint64_t)p->n_store;
    L.snap_stride = align_up(S * L.snap_shot);
    L.snap = take(L.snap_stride * dev_steps);
    L.ckpt_slot = L.set_bytes;
    L.ckpt = take(L.ckpt_slot * (uint64_t)p->n_ckpt);
    L.ev_row = (uint64_t)p->NS * (uint64_t)g.nx * 4;
    const uint64_t evb = L.ev_row * (uint64_t)p->EB;
    L.ev_fadd = take(evb);
    L.ev_fout = take(evb);
    L.ev_aadd = take(evb);
    L.ev_aout = take(evb);
    if (p->band_n > 0) {
        const uint64_t nw = (uint64_t)d.n_shots * (uint64_t)p->band_n;
        L.band_x_bytes = p->band_kx > 0
                             ? nw * 4 * (uint64_t)p->band_hd * (uint64_t)g.nx * BK_NW * 8   // [parity][side][7][hd][nx]
                             : nw * 8 * (uint64_t)g.P * (uint64_t)g.nx * 8;   // [kind][parity][side][P][nx] words
        L.band_x = take(L.band_x_bytes);
        L.band_err = take(4);
    }
    L.total = o;
    return true;
}

// Tiling of the step kernels over one device.  Strips are W columns wide;
// every (strip, shot) pair of the R = ny - 2P + 1 computed rows is cut into
// m chunks so that the grid is just below a whole number of "rounds" of the
// device's resident workgroups (cap) and chunks stay between 16 and chmax
// rows.  Small problems (fewer than two workgroups per CU) take short chunks
// instead (see below).  TM_FDTD_CHUNK_ROWS (environment, read when the
// tiling is made) forces the chunk height, for tuning.  ``small`` reports
// whether the small-problem rule chose the height.
Tiling make_tiling(const tm_desc& d, int P, int64_t cap, int W, int chmax = CH_MAX, int64_t ncu = 256,
                   int halo_iters = 0, bool* small = nullptr, bool allow_small = true)
{
    Tiling t{};
    const int R = (int)d.ny - 2 * P + 1, nx_e = (int)d.nx - 2 * P + 1;
    t.W = W;
    t.nstrip = (nx_e + W - 1) / W;
    const int64_t U = (int64_t)t.nstrip * d.n_shots;
    const int64_t m_max = std::max<int64_t>(1, (R + 15) / 16);
    int ch = R;
    for (int64_t k = 1; k <= 1 << 20; ++k) {
        const int64_t m = std::min<int64_t>(k * cap / U, m_max);
        if (m < 1) continue;
        ch = (int)((R + m - 1) / m);
        if (ch <= chmax) break;
    }
    ch = std::min(ch, chmax);
    // Small problems leave most CUs idle with chunks of 16 rows or more:
    // then each workgroup's time is its row count (owned rows plus the
    // halo_iters rows of its halo), so take the chunk height that minimises
    // (rows per workgroup) x (workgroups per pair of CUs, at least 1).
    const bool sm = allow_small && U * ((R + ch - 1) / ch) < 2 * ncu;
    if (sm) {
        double best = 1e300;
        for (int c = std::min(ch, chmax); c >= 1; --c) {
            const int64_t nblk = U * ((R + c - 1) / c);
            const double score = (double)(c + halo_iters) * std::max(1.0, (double)nblk / (2.0 * (double)ncu));
            if (score < best) { best = score; ch = c; }
        }
    }
    const char* env = std::getenv("TM_FDTD_CHUNK_ROWS");
    if (env != nullptr && std::atoi(env) >= 1) ch = std::min(std::atoi(env), chmax);
    if (small != nullptr) *small = sm || (env != nullptr && std::atoi(env) >= 1);
    t.CH = ch;
    t.nchunk = (R + ch - 1) / ch;
    t.nblk = (int)(U * t.nchunk);
    // the same cut in the two-step representation: equal weights, every
    // strip nchunk chunks of at most CH rows
    t.nbl = t.nbr = 0;
    t.nb_ch = t.ni_ch = t.nchunk;
    t.per_shot = t.nstrip * t.nchunk;
    t.wy0 = P;
    t.wy1 = P + R;
    t.wi = t.wb = 1;
    return t;
}

// Owned columns per strip of the two-step kernels: as many strips as
// columns of at most Strip2<P>::W need, cut to equal widths (so that no
// strip is a narrow, cheap remainder while the others set the time).
int strip2_width(int64_t nx, int P)
{
    const int nx_e = (int)nx - 2 * P + 1, w0 = NT - 8 * P + 4;
    const int n = (nx_e + w0 - 1) / w0;
    return (nx_e + n - 1) / n;
}

// Largest and smallest chunk height of a two-step cut into n chunks.
void chunk_heights(const Tiling& t, int ny, int P, int n, int& hmin, int& hmax)
{
    hmin = INT32_MAX;
    hmax = 0;
    int y = chunk_row(t, ny, P, 0, n);
    for (int k = 1; k <= n; ++k) {
        const int z = chunk_row(t, ny, P, k, n);
        hmin = std::min(hmin, z - y);
        hmax = std::max(hmax, z - y);
        y = z;
    }
}

// Tiling of the two-step kernels.  Large problems run a launch as a few
// rounds of resident workgroups, each of which streams its tile row by row
// at a rate set by memory latency; a launch ends with its slowest
// workgroups.  Rows on and near the y bands (CPML memories, predicated row
// blocks) cost about 1 + beta interior rows, and a strip with x-band lanes
// about mx times an interior strip.  Keeping the uniform tiling's rounds,
// this cut gives the band strips more, shorter chunks from the workgroups
// the uniform cut leaves unused, and cuts every strip at weighted row
// quantiles, so that band rows are spread over more tiles.
// TM_FDTD_BALANCE=0 keeps the uniform cut, =2 applies this one to small
// problems too (for tests).
Tiling make_tiling2(const tm_desc& d, const Geo& g, int P, int64_t cap, int W, int chmax, int64_t ncu,
                    int halo_iters, double beta, double mx, const char* tiles_env, bool* small_out = nullptr)
{
    const char* env = std::getenv("TM_FDTD_BALANCE");
    const int mode = env != nullptr ? std::atoi(env) : 1;
    bool small = false;
    Tiling t = make_tiling(d, P, cap, W, chmax, ncu, halo_iters, &small, mode != 2);
    if (small_out != nullptr) *small_out = small;
    t.W = strip2_width(d.nx, P);
    W = t.W;
    if (mode == 0 || small) return t;
    const int ny = (int)d.ny, R = ny - 2 * P + 1, S = (int)d.n_shots;
    const int64_t rounds = std::max<int64_t>(1, (t.nblk + cap - 1) / cap);
    const int64_t budget = rounds * cap / S;                     // tiles per shot
    if (budget < t.nstrip || budget > (int64_t)1 << 24) return t;
    // strips with x-band lanes (as the kernels decide it), from the edges in
    const int OFF = 4 * P - 2;
    auto band = [&](int st) {
        const int c0 = P + st * W - OFF;
        return c0 < g.x0 || c0 + NT - 1 >= g.hx1;
    };
    Tiling b = t;
    b.nbl = 0;
    while (b.nbl < t.nstrip && band(b.nbl)) ++b.nbl;
    b.nbr = 0;
    while (b.nbr < t.nstrip - b.nbl && band(t.nstrip - 1 - b.nbr)) ++b.nbr;
    const int nI = t.nstrip - b.nbl - b.nbr, nB = b.nbl + b.nbr;
    b.wi = 16;
    b.wb = 16 + (int)std::lround(16.0 * std::max(0.0, beta));
    b.wy0 = std::min(std::max(g.y0, P), P + R);
    b.wy1 = std::min(std::max(g.y1, b.wy0), P + R);
    const double tot = ((double)(b.wy0 - P) * b.wb + (double)(b.wy1 - b.wy0) * b.wi +
                        (double)(P + R - b.wy1) * b.wb) / b.wi;   // in interior rows
    auto cost = [&](int n, double m) { return m * (tot / n + halo_iters); };
    auto fits = [&](int n) {
        if (n < 1 || n > R) return false;
        int hmin = 0, hmax = 0;
        chunk_heights(b, ny, P, n, hmin, hmax);
        return hmin >= 1 && hmax <= chmax;
    };
    // Interior strips keep the uniform cut's chunk count (or the next one
    // whose weighted chunks fit); band strips take the count that brings
    // their tiles down to the interior tiles' cost, within the budget and
    // never fewer than the interior strips.  (Searching both counts by the
    // cost model alone chose fewer, longer interior chunks, which measured
    // slower.)
    int best_i = 0, best_b = 0;
    int64_t best_tiles = 0;
    int ni = nI > 0 ? std::max(1, t.nchunk) : 1;
    while (nI > 0 && ni <= R && (int64_t)nI * ni < budget && !fits(ni)) ++ni;
    if (nI == 0 || ((int64_t)nI * ni < budget && fits(ni))) {
        const double ci = nI > 0 ? cost(ni, 1.0) : 0.0;
        const int64_t left = budget - (int64_t)nI * ni;
        const int nb_max = nB > 0 ? (int)std::min<int64_t>(R, left / nB) : 1;
        int nb = 1;
        if (nB > 0) {
            const double room = ci / mx - halo_iters;
            nb = room > 0.0 ? (int)std::ceil(tot / room - 1e-9) : nb_max;
            nb = std::min(std::max(nb, nI > 0 ? ni : 1), nb_max);
            while (nb <= nb_max && !fits(nb)) ++nb;
        }
        if (nb >= 1 && nb <= nb_max && (nI == 0 || nb >= ni)) {
            best_i = ni;
            best_b = nb;
            best_tiles = (int64_t)nI * ni + (int64_t)nB * nb;
        }
    }
    // tiles_env = "ni,nb[,wb]" forces the chunk counts (and the band row
    // weight in 16ths), for tuning; ignored unless every chunk fits
    if (const char* e = std::getenv(tiles_env)) {
        int fi = 0, fb = 0, fw = b.wb;
        if (std::sscanf(e, "%d,%d,%d", &fi, &fb, &fw) >= 2 && fw >= 1) {
            Tiling f = b;
            f.wb = fw;
            int h0 = 0, h1 = 0, k0 = 0, k1 = 0;
            chunk_heights(f, ny, P, std::max(fi, 1), h0, h1);
            chunk_heights(f, ny, P, std::max(fb, 1), k0, k1);
            if (fi >= 1 && fb >= 1 && h0 >= 1 && h1 <= chmax && k0 >= 1 && k1 <= chmax) {
                b.wb = fw;
                best_i = fi;
                best_b = fb;
                best_tiles = (int64_t)nI * fi + (int64_t)nB * fb;
            }
        }
    }
    if (best_tiles == 0) return t;
    b.ni_ch = nI > 0 ? best_i : 1;
    b.nb_ch = nB > 0 ? best_b : 1;
    b.per_shot = (int)best_tiles;
    b.nblk = (int)(best_tiles * S);
    return b;
}

template <typename T>
T* wsp(void* ws, uint64_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

#define HIPCHK(expr)                                   \
    do {                                               \
        if ((expr) != hipSuccess) return TM_EHIP;      \
    } while (0)

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

hipEvent_t take_event(tm_plan* p)
{
    if (!p->ev_free.empty()) {
        hipEvent_t e = p->ev_free.back();
        p->ev_free.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Launch ``body`` (one kernel launch on ``st``), bracketed by a pair of
// events when this time step is sampled.
template <typename F>
void timed(tm_plan* p, int kid, int64_t t, hipStream_t st, F&& body)
{
    if (p->timing_every <= 0 || t % p->timing_every != 0) {
        body();
        return;
    }
    hipEvent_t a = take_event(p), b = take_event(p);
    if (a == nullptr || b == nullptr) {
        if (a) p->ev_free.push_back(a);
        if (b) p->ev_free.push_back(b);
        body();
        return;
    }
    (void)hipEventRecord(a, st);
    body();
    (void)hipEventRecord(b, st);
    p->ev_used.push_back(TimedLaunch{kid, a, b});
}

// Copies and zero fills gathered into k_fill launches (one per FILL_JOBS
// jobs), so that the small set-up work of a call costs one launch.
struct Fills {
    FillJobs j{};
    int count = 0;
    int64_t maxn = 0;
    tm_status launch(hipStream_t st)
    {
        if (count == 0) return TM_OK;
        for (int k = count; k < FILL_JOBS; ++k) {
            j.dst[k] = nullptr;
            j.src[k] = nullptr;
            j.n[k] = 0;
        }
        const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((maxn + 255) / 256, 8192));
        k_fill<<<dim3((unsigned)blocks, (unsigned)count), dim3(256), 0, st>>>(j);
        count = 0;
        maxn = 0;
        return hipGetLastError() == hipSuccess ? TM_OK : TM_EHIP;
    }
    // copy `bytes` from src (or zeros where src is null) to dst
    tm_status add(float* dst, const float* src, uint64_t bytes, hipStream_t st)
    {
        const int64_t n = (int64_t)(bytes / 4);
        if (n == 0) return TM_OK;
        if (count == FILL_JOBS) {
            const tm_status v = launch(st);
            if (v != TM_OK) return v;
        }
        j.dst[count] = dst;
        j.src[count] = src;
        j.n[count] = n;
        ++count;
        maxn = std::max(maxn, n);
        return TM_OK;
    }
};

// The plan's pinned read-back words and their event, made at first use.
constexpr int READBACK_WORDS = 1024;
tm_status ensure_readback(tm_plan* p)
{
    if (p->readback != nullptr) return TM_OK;
    HIPCHK(hipHostMalloc(reinterpret_cast<void**>(&p->readback), READBACK_WORDS * 4, hipHostMallocDefault));
    HIPCHK(hipEventCreateWithFlags(&p->readback_done, hipEventDisableTiming));
    return TM_OK;
}

// Wait for the work queued on st so far (a read-back copy into the pinned
// words at its end).  The host polls an event for up to SPIN_US
// microseconds, then blocks: a blocking wait alone wakes the host tens of
// microseconds after the device finishes, which the small problems (a few
// milliseconds per call) feel; a long wait does not keep a core busy.
constexpr int SPIN_US = 200;
tm_status wait_readback(tm_plan* p, hipStream_t st)
{
    HIPCHK(hipEventRecord(p->readback_done, st));
    const auto t0 = std::chrono::steady_clock::now();
    for (;;) {
        const hipError_t e = hipEventQuery(p->readback_done);
        if (e == hipSuccess) return TM_OK;
        if (e != hipErrorNotReady) return TM_EHIP;
        if (std::chrono::steady_clock::now() - t0 > std::chrono::microseconds(SPIN_US)) break;
    }
    HIPCHK(hipEventSynchronize(p->readback_done));
    return TM_OK;
}

tm_status zero(float* ptr, uint64_t bytes, hipStream_t st)
{
    const int64_t n = (int64_t)(bytes / 4);
    if (n == 0) return TM_OK;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 8192);
    k_zero<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(ptr, n);
    return hipGetLastError() == hipSuccess ? TM_OK : TM_EHIP;
}

tm_status upload_tables(tm_plan* p, void* ws, hipStream_t st)
{
    // the staging buffer mirrors the workspace from the CPML table to the
    // end of the event tables (which follow it), so one copy moves both
    const uint64_t cb = p->cpml.size() * 4, tb = p->tables.size() * 4;
    const uint64_t to = p->lay.tables - p->lay.cpml;
    if (p->pinned == nullptr) {
        p->pinned_bytes = to + tb;
        HIPCHK(hipHostMalloc(&p->pinned, p->pinned_bytes, hipHostMallocDefault));
        std::memset(p->pinned, 0, p->pinned_bytes);
        std::memcpy(p->pinned, p->cpml.data(), cb);
        if (tb) std::memcpy(static_cast<char*>(p->pinned) + to, p->tables.data(), tb);
    }
    HIPCHK(hipMemcpyAsync(wsp<char>(ws, p->lay.cpml), p->pinned, p->pinned_bytes, hipMemcpyHostToDevice, st));
    return TM_OK;
}

// Copy the caller's model arrays into the workspace's model block.
tm_status stage_model(tm_plan* p, void* ws, const float* ca, const float* cb, const float* cq, hipStream_t st,
                      Fills& fills)
{
    const uint64_t n = (uint64_t)p->g.slab * 4;
    char* m = wsp<char>(ws, p->lay.model);
    if (p->lay.model_stride == 0) {
        tm_status v = fills.add(reinterpret_cast<float*>(m), ca, n, st);
        if (v == TM_OK) v = fills.add(reinterpret_cast<float*>(m + p->lay.slab_b), cb, n, st);
        if (v == TM_OK) v = fills.add(reinterpret_cast<float*>(m + 2 * p->lay.slab_b), cq, n, st);
        return v;
    } else {                        // [S][ny][nx] each -> S blocks [Ca | Cb | Cq]
        const size_t S = (size_t)p->d.n_shots, pitch = (size_t)p->lay.model_stride;
        HIPCHK(hipMemcpy2DAsync(m, pitch, ca, n, n, S, hipMemcpyDeviceToDevice, st));
        HIPCHK(hipMemcpy2DAsync(m + p->lay.slab_b, pitch, cb, n, n, S, hipMemcpyDeviceToDevice, st));
        HIPCHK(hipMemcpy2DAsync(m + 2 * p->lay.slab_b, pitch, cq, n, n, S, hipMemcpyDeviceToDevice, st));
    }
    return TM_OK;
}

// Device pointers of one workspace.
struct Ptrs {
    char* base;
    const float* cp;
    Model model;
    const int32_t *row_slot, *colcell, *slot_shot, *cell_src, *src_list, *cell_rec, *rec_list, *src_pos, *rec_pos;
    float *ev_fadd, *ev_fout, *ev_aadd, *ev_aout;
    char *snap, *ckpt;
    float* scratch;
    uint64_t* band_x;                    // banded kernels: exchange rows
    int* band_err;                       // ... failure word
};

Ptrs pointers(const tm_plan* p, void* ws)
{
    const Layout& L = p->lay;
    Ptrs q{};
    q.base = static_cast<char*>(ws);
    q.cp = wsp<float>(ws, L.cpml);
    q.model = Model{wsp<char>(ws, L.model), (uint32_t)L.model_bytes, 0u, (uint32_t)L.slab_b,
                    (uint32_t)(2 * L.slab_b), (int64_t)L.model_stride};
    const int32_t* t = wsp<int32_t>(ws, L.tables);
    q.row_slot = t + p->t_slot; q.colcell = t + p->t_colcell; q.slot_shot = t + p->t_sshot;
    q.cell_src = t + p->t_cs; q.src_list = t + p->t_sl; q.cell_rec = t + p->t_cr; q.rec_list = t + p->t_rl;
    q.src_pos = t + p->t_spos; q.rec_pos = t + p->t_rpos;
    q.ev_fadd = wsp<float>(ws, L.ev_fadd); q.ev_fout = wsp<float>(ws, L.ev_fout);
    q.ev_aadd = wsp<float>(ws, L.ev_aadd); q.ev_aout = wsp<float>(ws, L.ev_aout);
    q.snap = wsp<char>(ws, L.snap);
    q.ckpt = wsp<char>(ws, L.ckpt);
    q.scratch = wsp<float>(ws, L.scratch);
    q.band_x = wsp<uint64_t>(ws, L.band_x);
    q.band_err = wsp<int>(ws, L.band_err);
    return q;
}

// Device destination of stored step t (t a multiple of R) in full-store
// mode: its own slot in the device store, or its ring slot in host mode.
int64_t dev_slot(const tm_plan* p, int64_t t)
{
    const int64_t j = t / p->R;
    return p->storage == TM_STORE_HOST ? j % HOST_RING : j;
}

tm_status host_setup(tm_plan* p)
{
    if (p->copy_stream == nullptr) HIPCHK(hipStreamCreateWithFlags(&p->copy_stream, hipStreamNonBlocking));
    for (int i = 0; i < HOST_RING; ++i) {
        if (p->slot_copied[i] == nullptr) HIPCHK(hipEventCreateWithFlags(&p->slot_copied[i], hipEventDisableTiming));
        if (p->slot_done[i] == nullptr) HIPCHK(hipEventCreateWithFlags(&p->slot_done[i], hipEventDisableTiming));
    }
    if (p->host_store == nullptr) {
        if (hipHostMalloc(reinterpret_cast<void**>(&p->host_store), p->host_bytes, hipHostMallocDefault) != hipSuccess) {
            p->host_store = nullptr;
            return TM_ENOMEM;
        }
    }
    return TM_OK;
}

// Before a kernel on `st` writes or reads ring slot i: wait for the slot's
// last copy.
tm_status slot_acquire(tm_plan* p, int i, hipStream_t st)
{
    if (p->slot_copy_pending[i]) HIPCHK(hipStreamWaitEvent(st, p->slot_copied[i], 0));
    p->slot_copy_pending[i] = false;
    return TM_OK;
}

// After the kernel that wrote / read ring slot i was enqueued on `st`.
tm_status slot_release(tm_plan* p, int i, hipStream_t st)
{
    HIPCHK(hipEventRecord(p->slot_done[i], st));
    p->slot_kernel_pending[i] = true;
    return TM_OK;
}

// Copy ring slot i to / from stored step j of the host store, after the
// slot's last kernel; the next kernel using the slot waits for it.
tm_status slot_copy(tm_plan* p, const Ptrs& q, int i, int64_t j, bool to_host)
{
    const uint64_t n = p->lay.snap_stride;
    hipStream_t cs = p->copy_stream;
    if (p->slot_kernel_pending[i]) HIPCHK(hipStreamWaitEvent(cs, p->slot_done[i], 0));
    p->slot_kernel_pending[i] = false;
    char* he = p->host_store + (uint64_t)j * n;          // the pairs of stored step j
    char* de = q.snap + (uint64_t)i * n;                 // the slot
    if (to_host) HIPCHK(hipMemcpyAsync(he, de, n, hipMemcpyDeviceToHost, cs));
    else HIPCHK(hipMemcpyAsync(de, he, n, hipMemcpyHostToDevice, cs));
    HIPCHK(hipEventRecord(p->slot_copied[i], cs));
    p->slot_copy_pending[i] = true;
    return TM_OK;
}

// Event-row view of the forward (adjoint = false) or adjoint buffers: the
// add rows [EB][NS][nx] followed by the out rows.
EventRows event_rows(const tm_plan* p, const Ptrs& q, bool adjoint)
{
    const Layout& L = p->lay;
    const uint64_t a = adjoint ? L.ev_aadd : L.ev_fadd, o = adjoint ? L.ev_aout : L.ev_fout;
    return EventRows{q.row_slot, q.base + a, (uint32_t)(o + L.ev_row * (uint64_t)p->EB - a)};
}

// Offsets of step t's add and out rows in that view.  Forward: add = the
// sources, out = the rows the receivers are gathered from; adjoint: add =
// the residual at the receivers, out = the rows of the source-wavelet
// gradient.
EventStep event_step(const tm_plan* p, bool adjoint, int64_t t)
{
    const Layout& L = p->lay;
    const uint64_t a = adjoint ? L.ev_aadd : L.ev_fadd, o = adjoint ? L.ev_aout : L.ev_fout;
    const uint64_t row = (uint64_t)(t % p->EB) * L.ev_row;
    return EventStep{(uint32_t)row, (uint32_t)(o - a + row)};
}

// One forward step t (set cur -> 1-cur): H and E updates, the step's
// sources and receivers and the snapshot epilogue (se/sc non-null) in one
// kernel.
template <int P>
void fwd_step(tm_plan* p, const Ptrs& q, int cur, float* r, int64_t t, int snap, char* sp, hipStream_t st)
{
    const Layout& L = p->lay;
    FwdArgs a;
    a.g = p->g;
    a.t = p->tiling_fwd;
    a.L = L.st;
    a.m = q.model;
    a.cp = q.cp;
    a.set0 = q.base + L.fset[cur];
    a.set1 = q.base + L.fset[1 - cur];
    a.snap = sp;
    a.snap_shot_bytes = (uint32_t)L.snap_shot;
    a.ev = event_rows(p, q, false);
    a.es = event_step(p, false, t);
    const dim3 grid((unsigned)p->tiling_fwd.nblk), blk(NT);
    timed(p, snap == SNAP_NONE ? KID_FWD_STEP : KID_FWD_STEP_ST, t, st, [&] {
        if (snap == SNAP_F32) k_fwd_step<P, SNAP_F32><<<grid, blk, 0, st>>>(a);
        else if (snap == SNAP_BF16) k_fwd_step<P, SNAP_BF16><<<grid, blk, 0, st>>>(a);
        else if (snap == SNAP_FP8) k_fwd_step<P, SNAP_FP8><<<grid, blk, 0, st>>>(a);
        else k_fwd_step<P, SNAP_NONE><<<grid, blk, 0, st>>>(a);
    });
}

// Forward steps t and t+1 in one launch (set cur -> 1-cur), with the
// sources and receivers of both.  sp0, sp1: snapshot destinations of
// steps t and t+1, or null.
template <int P>
void fwd_step2(tm_plan* p, const Ptrs& q, int cur, float* r, int64_t t, int snap, char* sp0, char* sp1,
               hipStream_t st)
{
    const Layout& L = p->lay;
    Fwd2Args a;
    a.g = p->g;
    a.t = p->tiling_fwd2;
    a.L = L.st;
    a.m = q.model;
    a.cp = q.cp;
    a.set0 = q.base + L.fset[cur];
    a.set1 = q.base + L.fset[1 - cur];
    a.snap0 = sp0;
    a.snap1 = sp1;
    a.snap_shot_bytes = (uint32_t)L.snap_shot;
    a.ev = event_rows(p, q, false);
    a.es0 = event_step(p, false, t);
    a.es1 = event_step(p, false, t + 1);
    a.cq = p->cq_value;
    const dim3 grid((unsigned)p->tiling_fwd2.nblk), blk(NT);
    const int kid = p->cq_uniform ? (snap == SNAP_NONE ? KID_FWD_STEP2_UQ : KID_FWD_STEP2_UQ_ST)
                                  : (snap == SNAP_NONE ? KID_FWD_STEP2 : KID_FWD_STEP2_ST);
    timed(p, kid, t, st, [&] {
        auto launch = [&](auto uq_t, auto cx_t) {
            constexpr bool UQ = decltype(uq_t)::value, CX = decltype(cx_t)::value;
            if (snap == SNAP_F32) k_fwd_step2<P, SNAP_F32, UQ, CX><<<grid, blk, 0, st>>>(a);
            else if (snap == SNAP_BF16) k_fwd_step2<P, SNAP_BF16, UQ, CX><<<grid, blk, 0, st>>>(a);
            else if (snap == SNAP_FP8) k_fwd_step2<P, SNAP_FP8, UQ, CX><<<grid, blk, 0, st>>>(a);
            else k_fwd_step2<P, SNAP_NONE, UQ, CX><<<grid, blk, 0, st>>>(a);
        };
        using T = std::true_type;
        using F = std::false_type;
        if constexpr (P == 4) {
            if (p->fwd_cx) {
                if (p->cq_uniform) launch(T{}, T{});
                else launch(F{}, T{});
                return;
            }
        }
        if (p->cq_uniform) launch(T{}, F{});
        else launch(F{}, F{});
    });
}

// One adjoint step t (residual injection at the receivers, transposed H and
// E updates, source-wavelet gradient and parameter-gradient accumulation in
// one kernel); k counts the adjoint launches (set k%2 -> (k+1)%2).
template <int P>
void adj_step(tm_plan* p, const Ptrs& q, int64_t t, int64_t k, int snap, const char* sp, float* gca,
              float* gcb, hipStream_t st)
{
    const Layout& L = p->lay;
    AdjArgs a;
    a.g = p->g;
    a.t = p->tiling_adj;
    a.L = L.st;
    a.m = q.model;
    a.cp = q.cp;
    a.set0 = q.base + L.aset[k & 1];
    a.set1 = q.base + L.aset[(k + 1) & 1];
    a.snap = sp;
    a.snap_shot_bytes = (uint32_t)L.snap_shot;
    a.gca = gca;
    a.gcb = gcb;
    a.ratio = (float)p->R;
    a.ev = event_rows(p, q, true);
    a.es = event_step(p, true, t);
    const dim3 grid((unsigned)p->tiling_adj.nblk), blk(NT);
    timed(p, KID_ADJ_STEP, t, st, [&] {
        if (snap == SNAP_F32) k_adj_step<P, SNAP_F32><<<grid, blk, 0, st>>>(a);
        else if (snap == SNAP_BF16) k_adj_step<P, SNAP_BF16><<<grid, blk, 0, st>>>(a);
        else if (snap == SNAP_FP8) k_adj_step<P, SNAP_FP8><<<grid, blk, 0, st>>>(a);
        else k_adj_step<P, SNAP_NONE><<<grid, blk, 0, st>>>(a);
    });
}

// Adjoint steps t and t-1 in one launch (set k%2 -> (k+1)%2, k counting
// launches); spA, spB: the snapshots of steps t and t-1, or null.
template <int P>
void adj_step2(tm_plan* p, const Ptrs& q, int64_t t, int64_t k, int snap, const char* spA, const char* spB,
               float* gca, float* gcb, hipStream_t st)
{
    const Layout& L = p->lay;
    Adj2Args a;
    a.g = p->g;
    a.t = p->tiling_adj2;
    a.L = L.st;
    a.m = q.model;
    a.cp = q.cp;
    a.set0 = q.base + L.aset[k & 1];
    a.set1 = q.base + L.aset[(k + 1) & 1];
    a.snapA = spA;
    a.snapB = spB;
    a.snap_shot_bytes = (uint32_t)L.snap_shot;
    a.gca = gca;
    a.gcb = gcb;
    a.ratio = (float)p->R;
    a.ev = event_rows(p, q, true);
    a.esA = event_step(p, true, t);
    a.esB = event_step(p, true, t - 1);
    a.cq = p->cq_value;
    const dim3 grid((unsigned)p->tiling_adj2.nblk), blk(NT);
    // sampled like the forward pairs (even step)
    timed(p, p->cq_uniform ? KID_ADJ_STEP2_UQ : KID_ADJ_STEP2, t - 1, st, [&] {
        if (p->cq_uniform) {
            if (snap == SNAP_F32) k_adj_step2<P, SNAP_F32, true><<<grid, blk, 0, st>>>(a);
            else if (snap == SNAP_BF16) k_adj_step2<P, SNAP_BF16, true><<<grid, blk, 0, st>>>(a);
            else if (snap == SNAP_FP8) k_adj_step2<P, SNAP_FP8, true><<<grid, blk, 0, st>>>(a);
            else k_adj_step2<P, SNAP_NONE, true><<<grid, blk, 0, st>>>(a);
        } else {
            if (snap == SNAP_F32) k_adj_step2<P, SNAP_F32, false><<<grid, blk, 0, st>>>(a);
            else if (snap == SNAP_BF16) k_adj_step2<P, SNAP_BF16, false><<<grid, blk, 0, st>>>(a);
            else if (snap == SNAP_FP8) k_adj_step2<P, SNAP_FP8, false><<<grid, blk, 0, st>>>(a);
            else k_adj_step2<P, SNAP_NONE, false><<<grid, blk, 0, st>>>(a);
        }
    });
}

// Forward steps [ta, tb) of one event block with the resident kernel (set
// cur -> 1-cur); stored steps go to the device store.
template <int P>
void fwd_small(tm_plan* p, const Ptrs& q, int cur, int64_t ta, int64_t tb, int snap, hipStream_t st)
{
    const Layout& L = p->lay;
    SmallArgs a{};
    a.g = p->g;
    a.L = L.st;
    a.m = q.model;
    a.cp = q.cp;
    a.set0 = q.base + L.fset[cur];
    a.set1 = q.base + L.fset[1 - cur];
    a.snap = snap != SNAP_NONE ? q.snap : nullptr;
    a.snap_stride = L.snap_stride;
    a.snap_shot_bytes = (uint32_t)L.snap_shot;
    a.R = (int)p->R;
    a.ratio = (float)p->R;
    a.t0 = (int)ta;
    a.t1 = (int)tb;
    a.ev = event_rows(p, q, false);
    const EventStep e0 = event_step(p, false, ta);
    a.ev_add0 = e0.add;
    a.ev_out0 = e0.out;
    a.ev_row = (uint32_t)L.ev_row;
    const uint32_t lds = small_lds_bytes(p->g, false);
    const dim3 grid((unsigned)p->d.n_shots), blk(NTS);
    timed(p, snap == SNAP_NONE ? KID_FWD_SMALL : KID_FWD_SMALL_ST, ta, st, [&] {
        if (snap == SNAP_F32) k_fwd_small<P, SNAP_F32><<<grid, blk, lds, st>>>(a);
        else if (snap == SNAP_BF16) k_fwd_small<P, SNAP_BF16><<<grid, blk, lds, st>>>(a);
        else if (snap == SNAP_FP8) k_fwd_small<P, SNAP_FP8><<<grid, blk, lds, st>>>(a);
        else k_fwd_small<P, SNAP_NONE><<<grid, blk, lds, st>>>(a);
    });
}

// Adjoint steps tb-1 .. ta of one event block with the resident kernel (set
// k%2 -> (k+1)%2); snapshots from the device store when snap is set.
template <int P>
void adj_small(tm_plan* p, const Ptrs& q, int64_t ta, int64_t tb, int64_t k, int snap, float* gca, float* gcb,
               hipStream_t st)
{
    const Layout& L = p->lay;
    SmallArgs a{};
    a.g = p->g;
    a.L = L.st;
    a.m = q.model;
    a.cp = q.cp;
    a.set0 = q.base + L.aset[k & 1];
    a.set1 = q.base + L.aset[(k + 1) & 1];
    a.snap = snap != SNAP_NONE ? q.snap : nullptr;
    a.snap_stride = L.snap_stride;
    a.snap_shot_bytes = (uint32_t)L.snap_shot;
    a.R = (int)p->R;
    a.ratio = (float)p->R;
    a.t0 = (int)ta;
    a.t1 = (int)tb;
    a.ev = event_rows(p, q, true);
    const EventStep e0 = event_step(p, true, ta);
    a.ev_add0 = e0.add;
    a.ev_out0 = e0.out;
    a.ev_row = (uint32_t)L.ev_row;
    a.gca = gca;
    a.gcb = gcb;
    const uint32_t lds = small_lds_bytes(p->g, true);
    const dim3 grid((unsigned)p->d.n_shots), blk(NTS);
    timed(p, KID_ADJ_SMALL, ta, st, [&] {
        if (snap == SNAP_F32) k_adj_small<P, SNAP_F32><<<grid, blk, lds, st>>>(a);
        else if (snap == SNAP_BF16) k_adj_small<P, SNAP_BF16><<<grid, blk, lds, st>>>(a);
        else if (snap == SNAP_FP8) k_adj_small<P, SNAP_FP8><<<grid, blk, lds, st>>>(a);
        else k_adj_small<P, SNAP_NONE><<<grid, blk, lds, st>>>(a);
    });
}

// Polls of one exchange wait before a banded launch counts as failed
// (about 0.2 s; a normal wait is a few microseconds).
constexpr int BAND_SPIN_MAX = 200000;

// The banded kernels' arguments for the run [ta, tb) on sets s0 -> s1.
BandArgs band_args(const tm_plan* p, const Ptrs& q, const SmallArgs& a)
{
    BandArgs b{};
    b.a = a;
    b.rb = p->band_rb;
    b.nband = p->band_n;
    b.xbuf = q.band_x;
    b.err = q.band_err;
    b.spin_max = BAND_SPIN_MAX;
    if (const char* e = std::getenv("TM_FDTD_BAND_SPIN")) b.spin_max = std::atoi(e);   // for tests
    return b;
}

// ... of the blocked banded kernels.
BandKArgs bandk_args(const tm_plan* p, const Ptrs& q, const SmallArgs& a)
{
    const BandArgs b = band_args(p, q, a);
    BandKArgs k{};
    k.a = a;
    k.rb = b.rb;
    k.nband = b.nband;
    k.hd = p->band_hd;
    k.kx = p->band_kx;
    k.xbuf = b.xbuf;
    k.err = b.err;
    k.spin_max = b.spin_max;
    return k;
}

// The blocked kernel instances of a snapshot format and cells per thread.
template <int P, int CK>
const void* fwd_bandk_fn(int snap)
{
    return snap == SNAP_F32    ? reinterpret_cast<const void*>(&k_fwd_bandk<P, SNAP_F32, CK>)
         : snap == SNAP_BF16   ? reinterpret_cast<const void*>(&k_fwd_bandk<P, SNAP_BF16, CK>)
         : snap == SNAP_FP8    ? reinterpret_cast<const void*>(&k_fwd_bandk<P, SNAP_FP8, CK>)
                               : reinterpret_cast<const void*>(&k_fwd_bandk<P, SNAP_NONE, CK>);
}
template <int P, int CK>
const void* adj_bandk_fn(int snap)
{
    return snap == SNAP_F32    ? reinterpret_cast<const void*>(&k_adj_bandk<P, SNAP_F32, CK>)
         : snap == SNAP_BF16   ? reinterpret_cast<const void*>(&k_adj_bandk<P, SNAP_BF16, CK>)
         : snap == SNAP_FP8    ? reinterpret_cast<const void*>(&k_adj_bandk<P, SNAP_FP8, CK>)
                               : reinterpret_cast<const void*>(&k_adj_bandk<P, SNAP_NONE, CK>);
}

// Launch a banded kernel cooperatively (all its workgroups resident at
// once), its exchange rows cleared first (their step tags restart at every
// launch); the failure word is cleared by the first banded launch of a call
// and read at the call's end.
tm_status band_launch(tm_plan* p, const Ptrs& q, const void* fn, void* argp, uint32_t lds, int kid, int64_t t,
                      hipStream_t st, int threads = NTS)
{
    const int nw = (int)(p->d.n_shots * p->band_n);
    Fills fills;
    tm_status v = fills.add(reinterpret_cast<float*>(q.band_x), nullptr, p->lay.band_x_bytes, st);
    if (v == TM_OK && !p->band_ran) v = fills.add(reinterpret_cast<float*>(q.band_err), nullptr, 4, st);
    if (v == TM_OK) v = fills.launch(st);
    if (v != TM_OK) return v;
    p->band_ran = true;
    void* args[] = {argp};
    hipError_t e = hipSuccess;
    timed(p, kid, t, st, [&] {
        e = hipLaunchCooperativeKernel(fn, dim3((unsigned)nw), dim3((unsigned)threads), args, lds, st);
    });
    return e == hipSuccess ? TM_OK : TM_EHIP;
}

// Whether the banded launches of this call completed every exchange (read
// back, so it waits for the stream; skipped while the stream is captured).
tm_status band_check(tm_plan* p, const Ptrs& q, hipStream_t st)
{
    if (!p->band_ran) return TM_OK;
    p->band_ran = false;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    HIPCHK(hipStreamIsCapturing(st, &cs));
    if (cs != hipStreamCaptureStatusNone) return TM_OK;
    tm_status v = ensure_readback(p);
    if (v != TM_OK) return v;
    HIPCHK(hipMemcpyAsync(p->readback, q.band_err, sizeof(int), hipMemcpyDeviceToHost, st));
    if ((v = wait_readback(p, st)) != TM_OK) return v;
    int failed = 0;
    std::memcpy(&failed, p->readback, sizeof(int));
    return failed ? TM_EHIP : TM_OK;
}

// Forward steps [ta, tb) of one event block with the banded kernels.
template <int P>
tm_status fwd_band(tm_plan* p, const Ptrs& q, int cur, int64_t ta, int64_t tb, int snap, hipStream_t st)
{
    const Layout& L = p->lay;
    SmallArgs a{};
    a.g = p->g;
    a.L = L.st;
    a.m = q.model;
    a.cp = q.cp;
    a.set0 = q.base + L.fset[cur];
    a.set1 = q.base + L.fset[1 - cur];
    a.snap = snap != SNAP_NONE ? q.snap : nullptr;
    a.snap_stride = L.snap_stride;
    a.snap_shot_bytes = (uint32_t)L.snap_shot;
    a.R = (int)p->R;
    a.ratio = (float)p->R;
    a.t0 = (int)ta;
    a.t1 = (int)tb;
    a.ev = event_rows(p, q, false);
    const EventStep e0 = event_step(p, false, ta);
    a.ev_add0 = e0.add;
    a.ev_out0 = e0.out;
    a.ev_row = (uint32_t)L.ev_row;
    if (p->band_kx > 0) {
        BandKArgs b = bandk_args(p, q, a);
        const void* fn = bandk_cells_per_thread(p->g, p->band_rb, p->band_hd) == 1 ? fwd_bandk_fn<P, 1>(snap)
                                                                                  : fwd_bandk_fn<P, CPTK>(snap);
        return band_launch(p, q, fn, &b, bandk_lds_bytes(p->g, p->band_rb, p->band_hd, false),
                           snap == SNAP_NONE ? KID_FWD_BANDK : KID_FWD_BANDK_ST, ta, st,
                           bandk_threads(p->g, p->band_rb, p->band_hd));
    }
    BandArgs b = band_args(p, q, a);
    const void* fn = snap == SNAP_F32    ? reinterpret_cast<const void*>(&k_fwd_band<P, SNAP_F32>)
                   : snap == SNAP_BF16   ? reinterpret_cast<const void*>(&k_fwd_band<P, SNAP_BF16>)
                   : snap == SNAP_FP8    ? reinterpret_cast<const void*>(&k_fwd_band<P, SNAP_FP8>)
                                         : reinterpret_cast<const void*>(&k_fwd_band<P, SNAP_NONE>);
    return band_launch(p, q, fn, &b, band_lds_bytes(p->g, p->band_rb, false),
                       snap == SNAP_NONE ? KID_FWD_BAND : KID_FWD_BAND_ST, ta, st);
}

// Adjoint steps tb-1 .. ta of one event block with the banded kernels.
template <int P>
tm_status adj_band(tm_plan* p, const Ptrs& q, int64_t ta, int64_t tb, int64_t k, int snap, float* gca, float* gcb,
                   hipStream_t st)
{
    const Layout& L = p->lay;
    SmallArgs a{};
    a.g = p->g;
    a.L = L.st;
    a.m = q.model;
    a.cp = q.cp;
    a.set0 = q.base + L.aset[k & 1];
    a.set1 = q.base + L.aset[(k + 1) & 1];
    a.snap = snap != SNAP_NONE ? q.snap : nullptr;
    a.snap_stride = L.snap_stride;
    a.snap_shot_bytes = (uint32_t)L.snap_shot;
    a.R = (int)p->R;
    a.ratio = (float)p->R;
    a.t0 = (int)ta;
    a.t1 = (int)tb;
    a.ev = event_rows(p, q, true);
    const EventStep e0 = event_step(p, true, ta);
    a.ev_add0 = e0.add;
    a.ev_out0 = e0.out;
    a.ev_row = (uint32_t)L.ev_row;
    a.gca = gca;
    a.gcb = gcb;
    if (p->band_kx > 0) {
        BandKArgs b = bandk_args(p, q, a);
        const void* fn = bandk_cells_per_thread(p->g, p->band_rb, p->band_hd) == 1 ? adj_bandk_fn<P, 1>(snap)
                                                                                  : adj_bandk_fn<P, CPTK>(snap);
        return band_launch(p, q, fn, &b, bandk_lds_bytes(p->g, p->band_rb, p->band_hd, true), KID_ADJ_BANDK, ta,
                           st, bandk_threads(p->g, p->band_rb, p->band_hd));
    }
    BandArgs b = band_args(p, q, a);
    const void* fn = snap == SNAP_F32    ? reinterpret_cast<const void*>(&k_adj_band<P, SNAP_F32>)
                   : snap == SNAP_BF16   ? reinterpret_cast<const void*>(&k_adj_band<P, SNAP_BF16>)
                   : snap == SNAP_FP8    ? reinterpret_cast<const void*>(&k_adj_band<P, SNAP_FP8>)
                                         : reinterpret_cast<const void*>(&k_adj_band<P, SNAP_NONE>);
    return band_launch(p, q, fn, &b, band_lds_bytes(p->g, p->band_rb, true), KID_ADJ_BAND, ta, st);
}

int snap_kind(const tm_plan* p)
{
    return p->d.snap == TM_SNAP_BF16 ? SNAP_BF16 : p->d.snap == TM_SNAP_FP8 ? SNAP_FP8 : SNAP_F32;
}

tm_status check_ws(const tm_plan* p, void* ws, uint64_t ws_bytes)
{
    if (ws == nullptr) return TM_EINVAL;
    if (ws_bytes < p->lay.total) return TM_ENOMEM;
    if ((reinterpret_cast<uintptr_t>(ws) & (ALIGN - 1)) != 0) return TM_EINVAL;
    return TM_OK;
}

// Resident workgroups of one step kernel on the current device.
// Target workgroups per CU for the step kernels: more resident workgroups
// than this only shorten the chunks (more halo rows re-read) without
// raising the bandwidth of this access pattern (measured on MI355X at the
// order-8, 1096^2 x 16-shot size: 5 per CU beat 4 and 7).
constexpr int WG_PER_CU = 5;

tm_status resident(const void* fn, int64_t* cap, int64_t* ncu_out = nullptr)
{
    int dev = 0, ncu = 0, nb = 0;
    HIPCHK(hipGetDevice(&dev));
    HIPCHK(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev));
    HIPCHK(hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, NT, 0));
    *cap = (int64_t)std::min(std::max(nb, 1), WG_PER_CU) * std::max(ncu, 1);
    if (ncu_out != nullptr) *ncu_out = std::max(ncu, 1);
    return TM_OK;
}

// Whether the x-band lanes of every strip of the two-step forward (strip
// width W) fit its compact FIFOs: the lanes with c < x0 or c >= hx1 inside
// the grid, counted as the kernel numbers them.
bool compact_xfifo_fits(const Geo& g, int P, int W, int nstrip)
{
    for (int st = 0; st < nstrip; ++st) {
        const int c0 = P + st * W - (4 * P - 2);
        const int cl = std::max(c0, 0), cr = std::max(g.hx1, c0);
        const int nl = std::max(0, std::min(g.x0, c0 + NT) - cl);
        const int nr = std::max(0, std::min(g.nx, c0 + NT) - cr);
        if (nl + nr > XFIFO_W) return false;
    }
    return true;
}

// Relative cost of a y-band row (1 + beta interior rows: the rows near the
// bands also leave the unrolled fast blocks) and of a strip with x-band
// lanes (mx interior strips) in the two-step kernels.  From per-workgroup
// timings and sweeps of the chunk counts and band weights on the order-8
// 1096^2 workload (16 shots), checked on the 4184^2 and order-4 428^2 ones.
constexpr double FWD2_BETA = 1.0, FWD2_MX = 1.14;
constexpr double ADJ2_BETA = 1.125, ADJ2_MX = 1.22;

// Make the tilings for the current device (once per device).
template <int P>
tm_status device_tiling(tm_plan* p)
{
    int dev = 0;
    HIPCHK(hipGetDevice(&dev));
    if (dev == p->tiling_device) return TM_OK;
    // occupancy of the storing instances (the ones the full step launches)
    auto pick = [&](auto f32, auto b16, auto f8) -> const void* {
        return p->d.snap == TM_SNAP_BF16 ? reinterpret_cast<const void*>(b16)
             : p->d.snap == TM_SNAP_FP8  ? reinterpret_cast<const void*>(f8)
                                         : reinterpret_cast<const void*>(f32);
    };
    int64_t cf = 0, ca = 0, c2 = 0, ncu = 0;
    tm_status v = resident(pick(&k_fwd_step<P, SNAP_F32>, &k_fwd_step<P, SNAP_BF16>, &k_fwd_step<P, SNAP_FP8>), &cf,
                           &ncu);
    if (v != TM_OK) return v;
    v = resident(pick(&k_adj_step<P, SNAP_F32>, &k_adj_step<P, SNAP_BF16>, &k_adj_step<P, SNAP_FP8>), &ca);
    if (v != TM_OK) return v;
    if constexpr (P == 4) {
        if (p->fwd_cx)
            v = resident(pick(&k_fwd_step2<P, SNAP_F32, false, true>, &k_fwd_step2<P, SNAP_BF16, false, true>,
                              &k_fwd_step2<P, SNAP_FP8, false, true>), &c2);
        else
            v = resident(pick(&k_fwd_step2<P, SNAP_F32, false, false>, &k_fwd_step2<P, SNAP_BF16, false, false>,
                              &k_fwd_step2<P, SNAP_FP8, false, false>), &c2);
    } else {
        v = resident(pick(&k_fwd_step2<P, SNAP_F32, false, false>, &k_fwd_step2<P, SNAP_BF16, false, false>,
                          &k_fwd_step2<P, SNAP_FP8, false, false>), &c2);
    }
    if (v != TM_OK) return v;
    int64_t ca2 = 0;
    v = resident(pick(&k_adj_step2<P, SNAP_F32, false>, &k_adj_step2<P, SNAP_BF16, false>,
                      &k_adj_step2<P, SNAP_FP8, false>), &ca2);
    if (v != TM_OK) return v;
    // halo_iters: row iterations of a chunk beyond its owned rows
    p->tiling_fwd = make_tiling(p->d, P, cf, Strip<P>::W, CH_MAX, ncu, 2 * P - 1);
    p->tiling_adj = make_tiling(p->d, P, ca, Strip<P>::W, CH_MAX, ncu, 4 * P - 3);
    bool stream_small = false;
    p->tiling_fwd2 = make_tiling2(p->d, p->g, P, c2, Strip2<P>::W, CH2_MAX, ncu, 6 * P - 3, FWD2_BETA, FWD2_MX,
                                   "TM_FDTD_FWD2_TILES", &stream_small);
    p->tiling_adj2 = make_tiling2(p->d, p->g, P, ca2, Strip2<P>::W, CHA2_MAX, ncu, 8 * P - 3, ADJ2_BETA, ADJ2_MX,
                                   "TM_FDTD_ADJ2_TILES");
    // resident kernels: the whole shot in one workgroup's LDS
    int lds_max = 0;
    HIPCHK(hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev));
    // (by default only with many shots: one workgroup, one CU, per shot is
    // slower than the streaming kernels spread over the device for a few
    // shots; measured on the 86^2 order-2 grid, the resident kernels win
    // from about 16 shots on)
    const bool fits = p->g.slab <= SMALL_CELLS && p->g.ny < 2048 && p->d.nt < (int64_t(1) << 30) &&
                      small_lds_bytes(p->g, false) <= (uint32_t)lds_max &&
                      small_lds_bytes(p->g, true) <= (uint32_t)lds_max;
    p->small = fits && (p->resident == 2 || (p->resident == 1 && p->d.n_shots >= SMALL_MIN_SHOTS));
    // banded resident kernels: where the streaming kernels would run a small
    // problem (few workgroups per CU) and every band's workgroup can be
    // resident at once
    p->banded = false;
    if (p->band_n > 0 && !p->small && (p->band == 2 || (p->band == 1 && stream_small))) {
        const bool kb = p->band_kx > 0;
        const uint32_t lf = kb ? bandk_lds_bytes(p->g, p->band_rb, p->band_hd, false)
                               : band_lds_bytes(p->g, p->band_rb, false);
        const uint32_t la = kb ? bandk_lds_bytes(p->g, p->band_rb, p->band_hd, true)
                               : band_lds_bytes(p->g, p->band_rb, true);
        if (lf <= (uint32_t)lds_max && la <= (uint32_t)lds_max) {
            int of = 0, oa = 0;
            const bool k1 = kb && bandk_cells_per_thread(p->g, p->band_rb, p->band_hd) == 1;
            const void* ff = !kb ? reinterpret_cast<const void*>(&k_fwd_band<P, SNAP_F32>)
                             : k1 ? fwd_bandk_fn<P, 1>(SNAP_F32) : fwd_bandk_fn<P, CPTK>(SNAP_F32);
            const void* fa = !kb ? reinterpret_cast<const void*>(&k_adj_band<P, SNAP_F32>)
                             : k1 ? adj_bandk_fn<P, 1>(SNAP_F32) : adj_bandk_fn<P, CPTK>(SNAP_F32);
            const int nth = kb ? bandk_threads(p->g, p->band_rb, p->band_hd) : NTS;
            HIPCHK(hipOccupancyMaxActiveBlocksPerMultiprocessor(&of, ff, nth, lf));
            HIPCHK(hipOccupancyMaxActiveBlocksPerMultiprocessor(&oa, fa, nth, la));
            p->banded = p->d.n_shots * p->band_n <= (int64_t)std::min(of, oa) * ncu;
        }
    }
    p->tiling_device = dev;
    return TM_OK;
}

// Event rows of the steps [ta, tb) (one event block): the sums of the
// step's inputs (f: sources, grad_r: receivers) into the add rows.
tm_status events_add(const tm_plan* p, const Ptrs& q, bool adjoint, const float* in, int64_t ta, int64_t tb,
                     hipStream_t st)
{
    const int64_t S = p->d.n_shots, n_in = adjoint ? p->d.n_rec : p->d.n_src;
    if (p->NS == 0 || tb <= ta) return TM_OK;           // (no inputs: rows of zeros)
    const int64_t n = (tb - ta) * p->NS * p->g.nx;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 8192);
    float* rows = (adjoint ? q.ev_aadd : q.ev_fadd) + (uint64_t)(ta % p->EB) * (p->lay.ev_row / 4);
    k_event_add<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(
        rows, n, (int)p->NS, p->g.nx, q.colcell, q.slot_shot, adjoint ? q.cell_rec : q.cell_src,
        adjoint ? q.rec_list : q.src_list, n_in > 0 ? in + ta * S * n_in : nullptr, (int)S, (int)n_in);
    return hipGetLastError() == hipSuccess ? TM_OK : TM_EHIP;
}

// Outputs of the steps [ta, tb) (one event block) from the out rows:
// receiver records (forward, into r) or the source-wavelet gradient
// (adjoint, into grad_f); absent entries get 0.
tm_status events_gather(const tm_plan* p, const Ptrs& q, bool adjoint, float* out, int64_t ta, int64_t tb,
                        hipStream_t st)
{
    const int64_t S = p->d.n_shots, n_out = adjoint ? p->d.n_src : p->d.n_rec;
    if (out == nullptr || n_out == 0 || tb <= ta) return TM_OK;
    const int64_t n = (tb - ta) * S * n_out;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 8192);
    const float* rows = (adjoint ? q.ev_aout : q.ev_fout) + (uint64_t)(ta % p->EB) * (p->lay.ev_row / 4);
    k_event_gather<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(
        out + ta * S * n_out, n, (int)(S * n_out), adjoint ? q.src_pos : q.rec_pos, rows,
        (int64_t)(p->lay.ev_row / 4));
    return hipGetLastError() == hipSuccess ? TM_OK : TM_EHIP;
}

// Forward steps [t0, t1) from set *cur (updated).  snap: SNAP_* kind of the
// stored steps (the multiples of R), whose device destinations
// snap_at(t) gives; host: copy every stored step to the host store
// through its ring slot; ckpt: save the state at every multiple of K into
// the checkpoint slots.
template <int P, typename SnapAt>
tm_status forward_range(tm_plan* p, const Ptrs& q, int* cur, const float* f, float* r, int64_t t0, int64_t t1,
                        int snap, SnapAt snap_at, bool ckpt, bool host, hipStream_t st)
{
    auto stored = [&](int64_t t) { return snap != SNAP_NONE && t % p->R == 0; };
    // the resident kernel runs each event block in one launch: snapshots in
    // the device store of full-store mode (not a replay's segment buffer),
    // or none; no checkpoints, no host store
    const bool small = p->small && !ckpt && !host && (p->K == 0 || snap == SNAP_NONE);
    const bool band = !small && p->banded && !ckpt && !host && (p->K == 0 || snap == SNAP_NONE);
    int64_t ev_a = t0, ev_b = t0;        // event block of the current steps: [ev_a, ev_b)
    tm_status v = TM_OK;
    for (int64_t t = t0; t < t1;) {
        if (t == ev_b) {                 // records of the finished block, add rows of the next
            if ((v = events_gather(p, q, false, r, ev_a, ev_b, st)) != TM_OK) return v;
            ev_a = t;
            ev_b = std::min(t1, (t / p->EB + 1) * p->EB);
            if ((v = events_add(p, q, false, f, ev_a, ev_b, st)) != TM_OK) return v;
        }
        if (small) {
            fwd_small<P>(p, q, *cur, t, ev_b, snap, st);
            *cur = 1 - *cur;
            t = ev_b;
            continue;
        }
        if (band) {
            if ((v = fwd_band<P>(p, q, *cur, t, ev_b, snap, st)) != TM_OK) return v;
            *cur = 1 - *cur;
            t = ev_b;
            continue;
        }
        if (ckpt && t > 0 && t % p->K == 0) {
            const int64_t slot = t / p->K - 1;
            HIPCHK(hipMemcpyAsync(q.ckpt + slot * p->lay.ckpt_slot, q.base + p->lay.fset[*cur],
                                  p->lay.ckpt_slot, hipMemcpyDeviceToDevice, st));
        }
        // two steps per launch unless step t+1 starts a checkpoint interval
        const bool pair = p->time_block == 2 && t + 1 < ev_b && !(ckpt && (t + 1) % p->K == 0);
        const int nstep = pair ? 2 : 1;
        char* sp[2] = {nullptr, nullptr};
        bool any = false;
        for (int i = 0; i < nstep; ++i) {
            if (!stored(t + i)) continue;
            sp[i] = snap_at(t + i);
            if (host) {
                tm_status v = slot_acquire(p, (int)dev_slot(p, t + i), st);
                if (v != TM_OK) return v;
            }
            any = true;
        }
        const int kind = any ? snap : SNAP_NONE;
        if (pair) fwd_step2<P>(p, q, *cur, r, t, kind, sp[0], sp[1], st);
        else fwd_step<P>(p, q, *cur, r, t, kind, sp[0], st);
        for (int i = 0; host && i < nstep; ++i) {
            if (!stored(t + i)) continue;
            const int slot = (int)dev_slot(p, t + i);
            tm_status v = slot_release(p, slot, st);
            if (v == TM_OK) v = slot_copy(p, q, slot, (t + i) / p->R, true);
            if (v != TM_OK) return v;
        }
        t += nstep;
        *cur = 1 - *cur;
    }
    if ((v = events_gather(p, q, false, r, ev_a, ev_b, st)) != TM_OK) return v;
    if (host) {                     // the caller's stream sees the host store complete
        for (int i = 0; i < HOST_RING; ++i) {
            if ((v = slot_acquire(p, i, st)) != TM_OK) return v;
        }
    }
    return hipGetLastError() == hipSuccess ? TM_OK : TM_EHIP;
}

template <int P>
tm_status run_forward(tm_plan* p, void* ws, const float* f, float* r, int64_t t0, int64_t t1, bool store,
                      hipStream_t st)
{
    tm_status v = device_tiling<P>(p);
    if (v != TM_OK) return v;
    const Ptrs q = pointers(p, ws);
    const bool full = p->K == 0;
    const int snap = (store && full) ? snap_kind(p) : SNAP_NONE;
    const bool host = snap != SNAP_NONE && p->storage == TM_STORE_HOST;
    if (host && (v = host_setup(p)) != TM_OK) return v;
    auto at = [&](int64_t t) { return q.snap + dev_slot(p, t) * p->lay.snap_stride; };
    return forward_range<P>(p, q, &p->fwd_cur, f, r, t0, t1, snap, at, store && !full, host, st);
}

template <int P>
tm_status run_adjoint(tm_plan* p, void* ws, const float* f, const float* grad_r, float* grad_f, float* gca,
                      float* gcb, hipStream_t st)
{
    tm_status v = device_tiling<P>(p);
    if (v != TM_OK) return v;
    const Ptrs q = pointers(p, ws);
    const int64_t nt = p->d.nt;
    const bool want_grad = gca != nullptr || gcb != nullptr;
    const int snap = want_grad ? snap_kind(p) : SNAP_NONE;
    int64_t k = 0;
    // Event blocks in reverse time: before the adjoint step t of a new
    // block [ev_a, ev_b), the source gradient of the finished block and the
    // residual rows of the new one.
    int64_t ev_a = nt, ev_b = nt;
    auto events = [&](int64_t t) {
        if (t >= ev_a) return TM_OK;
        tm_status e = events_gather(p, q, true, grad_f, ev_a, ev_b, st);
        if (e != TM_OK) return e;
        ev_b = t + 1;
        ev_a = (t / p->EB) * p->EB;
        return events_add(p, q, true, grad_r, ev_a, ev_b, st);
    };
    if (p->K == 0 || !want_grad) {
        const bool host = want_grad && p->storage == TM_STORE_HOST;
        const int64_t j_last = (nt - 1) / p->R;           // last stored step index
        if (host) {
            if ((v = host_setup(p)) != TM_OK) return v;
            for (int64_t j = j_last; j >= 0 && j > j_last - HOST_RING; --j)
                if ((v = slot_copy(p, q, (int)(j % HOST_RING), j, false)) != TM_OK) return v;
        }
        for (int64_t t = nt - 1; t >= 0; ++k) {
            if ((v = events(t)) != TM_OK) return v;
            if (p->small && !host) {                                           // the event block in one launch
                adj_small<P>(p, q, ev_a, t + 1, k, snap, gca, gcb, st);
                t = ev_a - 1;
                continue;
            }
            if (p->banded && !host) {                                          // ... with the banded kernels
                if ((v = adj_band<P>(p, q, ev_a, t + 1, k, snap, gca, gcb, st)) != TM_OK) return v;
                t = ev_a - 1;
                continue;
            }
            if (p->time_block == 2 && !host && t >= 1 && t - 1 >= ev_a) {   // steps t, t-1 in one launch
                const bool uA = want_grad && t % p->R == 0, uB = want_grad && (t - 1) % p->R == 0;
                const uint64_t oA = (uint64_t)(uA ? dev_slot(p, t) : 0) * p->lay.snap_stride;
                const uint64_t oB = (uint64_t)(uB ? dev_slot(p, t - 1) : 0) * p->lay.snap_stride;
                adj_step2<P>(p, q, t, k, (uA || uB) ? snap : SNAP_NONE, uA ? q.snap + oA : nullptr,
                             uB ? q.snap + oB : nullptr, gca, gcb, st);
                t -= 2;
                continue;
            }
            const bool use = want_grad && t % p->R == 0;
            const int64_t slot = use ? dev_slot(p, t) : 0;
            if (use && host && (v = slot_acquire(p, (int)slot, st)) != TM_OK) return v;
            const uint64_t so = (uint64_t)slot * p->lay.snap_stride;
            adj_step<P>(p, q, t, k, use ? snap : SNAP_NONE, use ? q.snap + so : nullptr, gca, gcb, st);
            if (use && host) {
                if ((v = slot_release(p, (int)slot, st)) != TM_OK) return v;
                const int64_t jn = t / p->R - HOST_RING;   // the stored step that reuses this slot
                if (jn >= 0 && (v = slot_copy(p, q, (int)slot, jn, false)) != TM_OK) return v;
            }
            --t;
        }
    } else {
        for (int64_t seg = p->n_seg - 1; seg >= 0; --seg) {
            const int64_t ta = seg * p->K, tb = std::min(ta + p->K, nt);
            // the segment's initial state into set 0
            if (seg == 0) {
                tm_status z = zero(wsp<float>(ws, p->lay.fwd), p->lay.fwd_bytes, st);
                if (z != TM_OK) return z;
            } else {
                HIPCHK(hipMemcpyAsync(q.base + p->lay.fset[0], q.ckpt + (seg - 1) * p->lay.ckpt_slot,
                                      p->lay.ckpt_slot, hipMemcpyDeviceToDevice, st));
            }
            int cur = 0;
            auto at = [&](int64_t t) { return q.snap + (t - ta) * p->lay.snap_stride; };
            v = forward_range<P>(p, q, &cur, f, nullptr, ta, tb, snap, at, false, false, st);
            if (v != TM_OK) return v;
            for (int64_t t = tb - 1; t >= ta; ++k) {
                if ((v = events(t)) != TM_OK) return v;
                const char* sp = q.snap + (t - ta) * p->lay.snap_stride;
                if (p->time_block == 2 && t - 1 >= ta && t - 1 >= ev_a) {
                    adj_step2<P>(p, q, t, k, snap, sp, sp - p->lay.snap_stride, gca, gcb, st);
                    t -= 2;
                } else {
                    adj_step<P>(p, q, t, k, snap, sp, gca, gcb, st);
                    --t;
                }
            }
        }
    }
    if ((v = events_gather(p, q, true, grad_f, ev_a, ev_b, st)) != TM_OK) return v;
    return hipGetLastError() == hipSuccess ? TM_OK : TM_EHIP;
}

// Event-row tables of the sources and receivers (validated indices) into
// the plan: the packed table block, the event-row count NS and the steps
// per event block EB.
tm_status set_events(tm_plan* p, const int64_t* src, const int64_t* rec)
{
    const tm_desc& d = p->d;
    std::vector<int32_t> tables;
    auto append = [&](const std::vector<int32_t>& v) {
        const uint64_t at = tables.size();
        tables.insert(tables.end(), v.begin(), v.end());
        return at;
    };
    const EventTables et = build_events(src, d.n_src, rec, d.n_rec, d.n_shots, d.ny, d.nx);
    if ((uint64_t)et.n_slots * (uint64_t)d.nx * 4 > EV_ROW_MAX) return TM_ENOMEM;
    p->t_slot = append(et.row_slot); p->t_colcell = append(et.colcell); p->t_sshot = append(et.slot_shot);
    p->t_cs = append(et.cell_src); p->t_sl = append(et.src_list);
    p->t_cr = append(et.cell_rec); p->t_rl = append(et.rec_list);
    p->t_spos = append(et.src_pos); p->t_rpos = append(et.rec_pos);
    p->tables = std::move(tables);
    p->NS = et.n_slots;
    // steps per event block: each of the four event buffers stays within
    // EV_BLOCK_BYTES; even, so that blocks do not split pairs of steps
    const int64_t eb_max = p->NS > 0 ? std::max<int64_t>(1, (int64_t)(EV_BLOCK_BYTES / (p->NS * d.nx * 4))) : d.nt;
    p->EB = std::min<int64_t>(d.nt, eb_max);
    if (p->EB > 1 && p->EB < d.nt) p->EB &= ~int64_t(1);
    if (const char* env = std::getenv("TM_FDTD_EVENT_STEPS")) {   // forced block length (tests, tuning)
        const long long v = std::atoll(env);
        if (v >= 1) p->EB = std::min<int64_t>(std::min<int64_t>(v, d.nt), eb_max);
    }
    return TM_OK;
}

// Per-block maxima of the Courant reduction and per-block flags of the
// uniform-Cq test, then cq[0]: the device scratch the check uses
// (COURANT_WORDS floats).
constexpr int COURANT_NB = 256;
constexpr int COURANT_WORDS = 2 * COURANT_NB + 1;
static_assert(COURANT_WORDS * sizeof(float) <= SCRATCH_BYTES, "Courant scratch exceeds the workspace's area");
static_assert(COURANT_WORDS <= READBACK_WORDS, "Courant read-back exceeds the plan's pinned words");

// scratch: COURANT_WORDS floats of device memory (the workspace's scratch
// area, or the static array of tm_courant_noalloc).
// pinned: read back through the plan's pinned words (a polled wait), else
// into host memory of the call (a blocking one; allocates nothing).
tm_status courant_impl(tm_plan* p, float* scratch, const float* cb, const float* cq, hipStream_t st, double* out,
                       bool pinned, bool* cq_one = nullptr, float* cq_val = nullptr)
{
    constexpr int NB = COURANT_NB;
    const int64_t n = p->g.slab * (p->d.model_per_shot ? p->d.n_shots : 1);   // every shot's model
    // per block: the largest cb*cq, whether Cq differs from cq[0]; cq[0]
    k_courant_scan<<<dim3(NB), dim3(256), 0, st>>>(cb, cq, n, scratch);
    HIPCHK(hipGetLastError());
    float part[COURANT_WORDS];
    if (pinned) {
        tm_status v = ensure_readback(p);
        if (v != TM_OK) return v;
        HIPCHK(hipMemcpyAsync(p->readback, scratch, sizeof(part), hipMemcpyDeviceToHost, st));
        if ((v = wait_readback(p, st)) != TM_OK) return v;
        std::memcpy(part, p->readback, sizeof(part));
    } else {
        HIPCHK(hipMemcpyAsync(part, scratch, sizeof(part), hipMemcpyDeviceToHost, st));
        HIPCHK(hipStreamSynchronize(st));
    }
    double m = 0.0;
    bool one = true;
    for (int i = 0; i < NB; ++i) {
        if (part[i] != part[i]) m = NAN;
        else if (m == m) m = std::max(m, (double)part[i]);
        one = one && part[NB + i] == 0.0f;
    }
    if (cq_one != nullptr) *cq_one = one;
    if (cq_val != nullptr) std::memcpy(cq_val, &part[2 * NB], sizeof(float));
    const double rdx = 1.0 / p->d.dx, rdy = 1.0 / p->d.dy;
    *out = std::sqrt(m) * abs_coef_sum(p->d.order) * std::sqrt(rdx * rdx + rdy * rdy);
    return TM_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

TM_API const char* tm_status_string(tm_status s)
{
    switch (s) {
    case TM_OK: return "ok";
    case TM_EINVAL: return "invalid argument";
    case TM_EUNSTABLE: return "unstable: Courant number above 1";
    case TM_ENOMEM: return "workspace too small or over the memory budget";
    case TM_EHIP: return "HIP runtime error";
    case TM_ESTATE: return "invalid call sequence";
    case TM_ENONFINITE: return "non-finite value";
    default: return "unknown status";
    }
}

TM_API tm_status tm_plan_create(const tm_desc* desc, const float* cpml, const int64_t* src,
                                const int64_t* rec, tm_plan** out)
{
    if (out == nullptr) return TM_EINVAL;
    *out = nullptr;
    if (desc == nullptr || cpml == nullptr) return TM_EINVAL;
    const tm_desc d = *desc;
    if (d.order != 2 && d.order != 4 && d.order != 8) return TM_EINVAL;
    const int P = d.order / 2;
    if (d.n_shots < 1 || d.nt < 1 || d.n_src < 0 || d.n_rec < 0 || d.ckpt_every < 0) return TM_EINVAL;
    if (d.snap != TM_SNAP_F32 && d.snap != TM_SNAP_BF16 && d.snap != TM_SNAP_FP8) return TM_EINVAL;
    if (d.time_block < 0 || d.time_block > 5) return TM_EINVAL;
    if (d.storage != TM_STORE_DEVICE && d.storage != TM_STORE_HOST) return TM_EINVAL;
    if (d.step_ratio < 0) return TM_EINVAL;
    if (d.model_per_shot != 0 && d.model_per_shot != 1) return TM_EINVAL;
    {
        const bool ckpt = d.ckpt_every > 0 && d.ckpt_every < d.nt;
        if (ckpt && (d.storage == TM_STORE_HOST || d.step_ratio > 1)) return TM_EINVAL;
    }
    if (d.ny < 2 * P + 2 || d.nx < 2 * P + 2) return TM_EINVAL;
    if (d.ny * d.nx >= (int64_t(1) << 29)) return TM_EINVAL;
    if (d.n_shots * std::max<int64_t>(d.n_src, d.n_rec) >= (int64_t(1) << 31)) return TM_EINVAL;
    if (d.n_shots > 65535) return TM_EINVAL;
    if (!(d.dy > 0.0) || !(d.dx > 0.0) || !std::isfinite(d.dy) || !std::isfinite(d.dx)) return TM_EINVAL;
    if (d.pml_y0 < P || d.pml_y1 <= d.pml_y0 || d.pml_y1 > d.ny - P + 1) return TM_EINVAL;
    if (d.pml_x0 < P || d.pml_x1 <= d.pml_x0 || d.pml_x1 > d.nx - P + 1) return TM_EINVAL;
    tm_status v = validate_indices(src, d.n_shots, d.n_src, d.ny, d.nx, P);
    if (v != TM_OK) return v;
    v = validate_indices(rec, d.n_shots, d.n_rec, d.ny, d.nx, P);
    if (v != TM_OK) return v;
    const int64_t L = std::max(d.ny, d.nx);
    if (!finite_all(cpml, 12 * L)) return TM_EINVAL;
    for (int64_t y = 0; y < d.ny; ++y) {
        if ((y < d.pml_y0 || y >= d.pml_y1 - 1) && (cpml[KY * L + y] == 0.0f || cpml[KYH * L + y] == 0.0f))
            return TM_EINVAL;
    }
    for (int64_t x = 0; x < d.nx; ++x) {
        if ((x < d.pml_x0 || x >= d.pml_x1 - 1) && (cpml[KX * L + x] == 0.0f || cpml[KXH * L + x] == 0.0f))
            return TM_EINVAL;
    }

    tm_plan* p = new (std::nothrow) tm_plan();
    if (p == nullptr) return TM_ENOMEM;
    p->d = d;
    p->P = P;
    Geo& g = p->g;
    g.ny = (int)d.ny; g.nx = (int)d.nx; g.P = P;
    g.y0 = (int)d.pml_y0; g.y1 = (int)d.pml_y1; g.x0 = (int)d.pml_x0; g.x1 = (int)d.pml_x1;
    g.hy1 = g.y1 - 1; g.hx1 = g.x1 - 1;
    g.byl = g.y0; g.by = g.y0 + (g.ny - g.hy1);
    g.bxl = g.x0; g.bx = g.x0 + (g.nx - g.hx1);
    g.nyi = g.y1 - g.y0; g.nxi = g.x1 - g.x0;
    g.L = (int)L;
    g.rdy = (float)(1.0 / d.dy); g.rdx = (float)(1.0 / d.dx);
    g.slab = d.ny * d.nx;
    p->cpml.assign(cpml, cpml + 12 * L);

    if ((v = set_events(p, src, rec)) != TM_OK) { delete p; return v; }
    p->time_block = (d.time_block == 0 || d.time_block >= 3) ? 2 : (int)d.time_block;
    p->resident = d.time_block == 0 ? 1 : d.time_block == 3 ? 2 : 0;
    p->band = d.time_block == 0 ? 1 : (d.time_block == 4 || d.time_block == 5) ? 2 : 0;
    {
        // blocked banded kernels: asked for (time_block 5), and by default
        // at order 2, where the halo of a step is one row
        int kx = d.time_block == 5 || (d.time_block == 0 && P == 1) ? BANDK_STEPS : 0;
        if (const char* e = std::getenv("TM_FDTD_BAND_KX")) kx = std::max(0, std::atoi(e));   // tuning, tests
        band_plan(p, kx);
    }
    p->R = d.step_ratio > 1 ? d.step_ratio : 1;
    p->n_store = (d.nt + p->R - 1) / p->R;
    p->storage = (int)d.storage;

    if (d.ckpt_every > 0 && d.ckpt_every < d.nt) {
        p->K = d.ckpt_every;
        p->n_seg = (d.nt + p->K - 1) / p->K;
        p->n_ckpt = p->n_seg - 1;
        p->seg_steps = p->K;
    } else {
        p->K = 0;
        p->n_seg = 1;
        p->n_ckpt = 0;
        p->seg_steps = d.nt;
    }
    p->tiling_fwd = p->tiling_adj = make_tiling(d, P, 1024, NT - 4 * P + 2);
    p->tiling_fwd2 = make_tiling(d, P, 1024, NT - 8 * P + 4, CH2_MAX);
    p->tiling_fwd2.W = strip2_width(d.nx, P);
    p->fwd_cx = P == 4 && compact_xfifo_fits(p->g, P, p->tiling_fwd2.W, p->tiling_fwd2.nstrip);
    p->tiling_adj2 = make_tiling(d, P, 1024, NT - 8 * P + 4, CHA2_MAX);
    p->tiling_adj2.W = strip2_width(d.nx, P);
    if (!make_layout(p)) {
        delete p;
        return TM_EINVAL;
    }
    if (p->storage == TM_STORE_HOST) p->host_bytes = (uint64_t)p->n_store * p->lay.snap_stride;
    if (d.hbm_budget > 0 && p->lay.total > d.hbm_budget) {
        delete p;
        return TM_ENOMEM;
    }
    *out = p;
    return TM_OK;
}

TM_API tm_status tm_plan_set_indices(tm_plan* p, const int64_t* src, const int64_t* rec)
{
    if (p == nullptr) return TM_EINVAL;
    const tm_desc& d = p->d;
    tm_status v = validate_indices(src, d.n_shots, d.n_src, d.ny, d.nx, p->P);
    if (v != TM_OK) return v;
    if ((v = validate_indices(rec, d.n_shots, d.n_rec, d.ny, d.nx, p->P)) != TM_OK) return v;
    // what the new tables replace, restored when they do not fit
    struct Saved {
        std::vector<int32_t> tables;
        uint64_t off[9];
        int64_t NS, EB;
        Layout lay;
    } old{p->tables, {p->t_slot, p->t_colcell, p->t_sshot, p->t_cs, p->t_sl, p->t_cr, p->t_rl, p->t_spos,
                      p->t_rpos}, p->NS, p->EB, p->lay};
    auto restore = [&] {
        p->tables = std::move(old.tables);
        p->t_slot = old.off[0]; p->t_colcell = old.off[1]; p->t_sshot = old.off[2]; p->t_cs = old.off[3];
        p->t_sl = old.off[4]; p->t_cr = old.off[5]; p->t_rl = old.off[6]; p->t_spos = old.off[7];
        p->t_rpos = old.off[8];
        p->NS = old.NS;
        p->EB = old.EB;
        p->lay = old.lay;
    };
    v = set_events(p, src, rec);
    if (v == TM_OK && !make_layout(p)) v = TM_EINVAL;
    if (v == TM_OK && d.hbm_budget > 0 && p->lay.total > d.hbm_budget) v = TM_ENOMEM;
    if (v == TM_OK && p->pinned != nullptr) {
        // earlier calls may still be copying the old tables from the pinned
        // staging buffer: wait for the device before freeing it
        if (hipDeviceSynchronize() != hipSuccess) v = TM_EHIP;
    }
    if (v != TM_OK) {
        restore();
        return v;
    }
    if (p->pinned != nullptr) {
        (void)hipHostFree(p->pinned);
        p->pinned = nullptr;            // restaged at the next device call
    }
    // the workspace's state belongs to the old geometry
    p->ws_last = nullptr;
    p->fwd_next = -1;
    p->stored_ok = false;
    p->fwd_complete = false;
    return TM_OK;
}

TM_API void tm_plan_destroy(tm_plan* p)
{
    if (p == nullptr) return;
    if (p->pinned != nullptr) (void)hipHostFree(p->pinned);
    if (p->readback_done != nullptr) (void)hipEventSynchronize(p->readback_done);
    if (p->readback != nullptr) (void)hipHostFree(p->readback);
    if (p->readback_done != nullptr) (void)hipEventDestroy(p->readback_done);
    if (p->copy_stream != nullptr) (void)hipStreamSynchronize(p->copy_stream);
    if (p->host_store != nullptr) (void)hipHostFree(p->host_store);
    if (p->copy_stream != nullptr) (void)hipStreamDestroy(p->copy_stream);
    for (int i = 0; i < HOST_RING; ++i) {
        if (p->slot_copied[i] != nullptr) (void)hipEventDestroy(p->slot_copied[i]);
        if (p->slot_done[i] != nullptr) (void)hipEventDestroy(p->slot_done[i]);
    }
    for (const TimedLaunch& r : p->ev_used) {
        (void)hipEventSynchronize(r.b);
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
    }
    for (hipEvent_t e : p->ev_free) (void)hipEventDestroy(e);
    delete p;
}

TM_API tm_status tm_timing_enable(tm_plan* p, int32_t every)
{
    if (p == nullptr || every < 0) return TM_EINVAL;
    p->timing_every = every;
    return TM_OK;
}

TM_API tm_status tm_timing_read(tm_plan* p, double* total_ms, int64_t* count)
{
    if (p == nullptr || total_ms == nullptr || count == nullptr) return TM_EINVAL;
    tm_status rc = TM_OK;
    for (const TimedLaunch& r : p->ev_used) {
        float ms = 0.0f;
        if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
            rc = TM_EHIP;
        } else {
            p->t_ms[r.kid] += ms;
            p->t_n[r.kid] += 1;
        }
        p->ev_free.push_back(r.a);
        p->ev_free.push_back(r.b);
    }
    p->ev_used.clear();
    for (int k = 0; k < KID_COUNT; ++k) {
        total_ms[k] = p->t_ms[k];
        count[k] = p->t_n[k];
        p->t_ms[k] = 0.0;
        p->t_n[k] = 0;
    }
    return rc;
}

TM_API int32_t tm_kernel_count(void) { return KID_COUNT; }

TM_API const char* tm_kernel_name(int32_t k)
{
    return (k >= 0 && k < KID_COUNT) ? KERNEL_NAMES[k] : nullptr;
}

TM_API tm_status tm_workspace_bytes(const tm_plan* p, uint64_t* bytes)
{
    if (p == nullptr || bytes == nullptr) return TM_EINVAL;
    *bytes = p->lay.total;
    return TM_OK;
}

TM_API tm_status tm_courant(tm_plan* p, void* ws, uint64_t ws_bytes, const float* cb, const float* cq,
                            void* stream, double* courant)
{
    if (p == nullptr || cb == nullptr || cq == nullptr || courant == nullptr) return TM_EINVAL;
    tm_status v = check_ws(p, ws, ws_bytes);
    if (v != TM_OK) return v;
    return courant_impl(p, pointers(p, ws).scratch, cb, cq, as_stream(stream), courant, true);
}

// ---------------------------------------------------------------------------
// tm_courant_noalloc: the Courant check with its scratch in static device
// memory, for callers that cannot allocate (and before a workspace exists).
// Every device the library runs on holds one copy of the array until the
// process ends; host code reaches it only through the address that
// hipGetSymbolAddress returns on that device (the array's name is a host
// stand-in).  Calls that overlap on one device share the array and race.
// ---------------------------------------------------------------------------

static __device__ __align__(256) float noalloc_scratch[COURANT_WORDS];

namespace {
constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex noalloc_mu;
float* noalloc_ptr[NOALLOC_MAX_DEVICES] = {};

// The device address of the current device's copy of noalloc_scratch,
// looked up once per device.
tm_status noalloc_scratch_ptr(float** out)
{
    int dev = 0;
    HIPCHK(hipGetDevice(&dev));
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return TM_EINVAL;
    std::lock_guard<std::mutex> lock(noalloc_mu);
    if (noalloc_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(noalloc_scratch)) != hipSuccess || ptr == nullptr) return TM_EHIP;
        noalloc_ptr[dev] = static_cast<float*>(ptr);
    }
    *out = noalloc_ptr[dev];
    return TM_OK;
}
}  // namespace

TM_API tm_status tm_courant_noalloc(tm_plan* p, const float* cb, const float* cq, void* stream, double* courant)
{
    if (p == nullptr || cb == nullptr || cq == nullptr || courant == nullptr) return TM_EINVAL;
    float* scratch = nullptr;
    tm_status v = noalloc_scratch_ptr(&scratch);
    if (v != TM_OK) return v;
    return courant_impl(p, scratch, cb, cq, as_stream(stream), courant, false);
}

TM_API tm_status tm_forward(tm_plan* p, void* ws, uint64_t ws_bytes, const float* ca, const float* cb,
                            const float* cq, const float* f, float* r, int64_t t0, int64_t t1,
                            int32_t flags, void* stream)
{
    if (p == nullptr || ca == nullptr || cb == nullptr || cq == nullptr) return TM_EINVAL;
    if (p->d.n_src > 0 && f == nullptr) return TM_EINVAL;
    if (t0 < 0 || t1 <= t0 || t1 > p->d.nt) return TM_EINVAL;
    if ((flags & ~(TM_FWD_STORE | TM_FWD_CHECK)) != 0) return TM_EINVAL;
    tm_status v = check_ws(p, ws, ws_bytes);
    if (v != TM_OK) return v;
    if (t0 > 0 && (ws != p->ws_last || p->fwd_next != t0)) return TM_ESTATE;
    hipStream_t st = as_stream(stream);
    const bool store = (flags & TM_FWD_STORE) != 0;
    bool cq_one = false;
    float cq_val = 0.0f;
    if (flags & TM_FWD_CHECK) {
        double c = 0.0;
        v = courant_impl(p, pointers(p, ws).scratch, cb, cq, st, &c, true, &cq_one, &cq_val);
        if (v != TM_OK) return v;
        if (!(c <= 1.0)) return TM_EUNSTABLE;
    }
    if ((v = upload_tables(p, ws, st)) != TM_OK) return v;
    Fills fills;
    if ((v = stage_model(p, ws, ca, cb, cq, st, fills)) != TM_OK) return v;
    if (t0 == 0 && (v = fills.add(wsp<float>(ws, p->lay.fwd), nullptr, p->lay.fwd_bytes, st)) != TM_OK) return v;
    if ((v = fills.launch(st)) != TM_OK) return v;
    if (t0 == 0) {
        p->fwd_complete = false;
        p->fwd_cur = 0;
        p->stored_ok = store;
    } else {
        p->stored_ok = p->stored_ok && store;
    }
    p->ws_last = ws;
    p->fwd_next = -1;
    if (t0 == 0) {
        p->fwd_cq = cq;
        p->fwd_cq_one = cq_one;
        p->fwd_cq_val = cq_val;
    } else {
        p->fwd_cq_one = p->fwd_cq_one && cq_one && cq == p->fwd_cq &&
                        std::memcmp(&cq_val, &p->fwd_cq_val, sizeof(float)) == 0;
    }
    p->cq_uniform = cq_one;
    p->cq_value = cq_val;
    switch (p->P) {
    case 1: v = run_forward<1>(p, ws, f, r, t0, t1, store, st); break;
    case 2: v = run_forward<2>(p, ws, f, r, t0, t1, store, st); break;
    default: v = run_forward<4>(p, ws, f, r, t0, t1, store, st); break;
    }
    p->cq_uniform = false;            // the adjoint's replays read the array
    if (v == TM_OK) v = band_check(p, pointers(p, ws), st);
    p->band_ran = false;
    if (v != TM_OK) return v;
    p->fwd_next = t1;
    p->fwd_complete = (t1 == p->d.nt) && p->stored_ok;
    return TM_OK;
}

TM_API tm_status tm_adjoint(tm_plan* p, void* ws, uint64_t ws_bytes, const float* ca, const float* cb,
                            const float* cq, const float* f, const float* grad_r, float* grad_f,
                            float* grad_ca_shot, float* grad_cb_shot, void* stream)
{
    if (p == nullptr || ca == nullptr || cb == nullptr || cq == nullptr) return TM_EINVAL;
    if (p->d.n_rec > 0 && grad_r == nullptr) return TM_EINVAL;
    tm_status v = check_ws(p, ws, ws_bytes);
    if (v != TM_OK) return v;
    const bool want_grad = grad_ca_shot != nullptr || grad_cb_shot != nullptr;
    if (want_grad) {
        if (ws != p->ws_last || !p->fwd_complete) return TM_ESTATE;
        if (p->K > 0 && p->d.n_src > 0 && f == nullptr) return TM_EINVAL;
    }
    hipStream_t st = as_stream(stream);
    // after the storing forward on this workspace (whose snapshots the
    // gradients read) the tables it uploaded are still there
    if (!want_grad && (v = upload_tables(p, ws, st)) != TM_OK) return v;
    Fills fills;
    if ((v = stage_model(p, ws, ca, cb, cq, st, fills)) != TM_OK) return v;
    if ((v = fills.add(wsp<float>(ws, p->lay.adj), nullptr, p->lay.adj_bytes, st)) != TM_OK) return v;
    const uint64_t gbytes = (uint64_t)p->d.n_shots * (uint64_t)p->g.slab * 4;
    if (grad_ca_shot && (v = fills.add(grad_ca_shot, nullptr, gbytes, st)) != TM_OK) return v;
    if (grad_cb_shot && (v = fills.add(grad_cb_shot, nullptr, gbytes, st)) != TM_OK) return v;
    if ((v = fills.launch(st)) != TM_OK) return v;
    // the adjoint steps and the checkpoint replays take the arrays of the
    // storing forward: its check's finding holds for them
    p->cq_uniform = p->fwd_cq_one && cq == p->fwd_cq;
    p->cq_value = p->fwd_cq_val;
    switch (p->P) {
    case 1: v = run_adjoint<1>(p, ws, f, grad_r, grad_f, grad_ca_shot, grad_cb_shot, st); break;
    case 2: v = run_adjoint<2>(p, ws, f, grad_r, grad_f, grad_ca_shot, grad_cb_shot, st); break;
    default: v = run_adjoint<4>(p, ws, f, grad_r, grad_f, grad_ca_shot, grad_cb_shot, st); break;
    }
    p->cq_uniform = false;
    if (v == TM_OK) v = band_check(p, pointers(p, ws), st);
    p->band_ran = false;
    if (v != TM_OK) return v;
    if (p->K > 0 && want_grad) p->fwd_next = -1;   // the replay overwrote the forward state
    return TM_OK;
}

TM_API tm_status tm_grad(const tm_plan* p, const float* grad_ca_shot, const float* grad_cb_shot,
                         float* grad_ca, float* grad_cb, void* stream)
{
    if (p == nullptr) return TM_EINVAL;
    if ((grad_ca == nullptr) != (grad_ca_shot == nullptr)) return TM_EINVAL;
    if ((grad_cb == nullptr) != (grad_cb_shot == nullptr)) return TM_EINVAL;
    hipStream_t st = as_stream(stream);
    const int64_t slab = p->g.slab;
    // the requested sums in one launch: pair 0 the first requested, pair 1 the other
    const float* gs[2] = {nullptr, nullptr};
    float* out[2] = {nullptr, nullptr};
    int n = 0;
    if (grad_ca) { gs[n] = grad_ca_shot; out[n] = grad_ca; ++n; }
    if (grad_cb) { gs[n] = grad_cb_shot; out[n] = grad_cb; ++n; }
    if (n == 0) return TM_OK;
    const dim3 grid((unsigned)((slab + 255) / 256), (unsigned)n), blk(256);
    k_shot_sum<<<grid, blk, 0, st>>>(slab, (int)p->d.n_shots, gs[0], out[0], gs[1], out[1]);
    return hipGetLastError() == hipSuccess ? TM_OK : TM_EHIP;
}

TM_API tm_status tm_grad_eps_sigma(const tm_plan* p, const float* ca, const float* cb, const float* grad_ca,
                                   const float* grad_cb, double dt, float* grad_eps_r, float* grad_sigma,
                                   void* stream)
{
    if (p == nullptr || ca == nullptr || cb == nullptr) return TM_EINVAL;
    if (!(dt > 0.0) || !std::isfinite(dt) || !std::isfinite(1.0 / dt)) return TM_EINVAL;
    if (grad_eps_r == nullptr && grad_sigma == nullptr) return TM_OK;
    hipStream_t st = as_stream(stream);
    const int64_t n = p->g.slab;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
    k_eps_sigma<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(n, ca, cb, grad_ca, grad_cb, (float)(1.0 / dt),
                                                             grad_eps_r, grad_sigma);
    return hipGetLastError() == hipSuccess ? TM_OK : TM_EHIP;
}

TM_API tm_status tm_fp8_encode(const float* in, uint8_t* out, int64_t n, void* stream)
{
    if (n < 0 || (n > 0 && (in == nullptr || out == nullptr))) return TM_EINVAL;
    if (n == 0) return TM_OK;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
    k_fp8_encode<<<dim3((unsigned)blocks), dim3(256), 0, as_stream(stream)>>>(in, out, n);
    return hipGetLastError() == hipSuccess ? TM_OK : TM_EHIP;
}

TM_API tm_status tm_fp8_decode(const uint8_t* in, float* out, int64_t n, void* stream)
{
    if (n < 0 || (n > 0 && (in == nullptr || out == nullptr))) return TM_EINVAL;
    if (n == 0) return TM_OK;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
    k_fp8_decode<<<dim3((unsigned)blocks), dim3(256), 0, as_stream(stream)>>>(in, out, n);
    return hipGetLastError() == hipSuccess ? TM_OK : TM_EHIP;
}
