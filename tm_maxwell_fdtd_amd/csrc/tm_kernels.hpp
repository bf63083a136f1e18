// HIP kernels of the TM FDTD forward step, its exact adjoint and the
// gradient shot sum (gfx950, wave64).
//
// Forward (tide maxwell.cu, forward_kernel_h / forward_kernel_e): two
// in-place passes per step.  The H pass reads only Ey and writes Hx, Hz;
// the E pass reads only Hx, Hz and writes Ey, so both are race-free.
//
// Adjoint: the exact transpose of the forward step (the page's header
// comment: time-reversed, transposed operators), CPML included.  Per step:
//   band pre-pass  : on E cells in a CPML band, run the E-update filters
//                    backwards on Cb*lambda_E (own adjoint memories) and keep
//                    the filtered values in band-only buffers;
//   lambda_H pass  : lambda_Hz -= Dx^h[u], lambda_Hx += Dz^h[w] where u, w are
//                    Cb*lambda_E off the band and the filtered values on it;
//                    then, on H cells in a band, filter Cq*lambda_H backwards
//                    and keep the results in band-only buffers;
//   lambda_E pass  : gradients (interior only), then
//                    lambda_E = Ca*lambda_E - Dx[t_z] + Dz[t_x] with t = Cq*lambda_H
//                    off the band and the filtered values on it.
// Every cell has exactly one writer per pass; there are no atomics.
#pragma once

#include "tm_common.hpp"

namespace tmf {

constexpr int BLK_X = 64;   // one wave64 along a row
constexpr int BLK_Y = 4;

// ---------------------------------------------------------------------------
// Forward H half-step: Hx -= Cq * filt(Dz^h Ey), Hz += Cq * filt(Dx^h Ey)
// ---------------------------------------------------------------------------
template <int P>
__global__ __launch_bounds__(BLK_X* BLK_Y) void k_fwd_h(Geo g, const float* __restrict__ cq,
                                                        const float* __restrict__ E,
                                                        float* __restrict__ Hx, float* __restrict__ Hz,
                                                        float* __restrict__ psi_ez,
                                                        float* __restrict__ psi_ex,
                                                        const float* __restrict__ cp)
{
    const int x = blockIdx.x * BLK_X + threadIdx.x + P;
    const int y = blockIdx.y * BLK_Y + threadIdx.y + P;
    const int s = blockIdx.z;
    if (x > g.nx - P || y > g.ny - P) return;
    const int nx = g.nx;
    const int64_t base = (int64_t)s * g.slab;
    const float* e = E + base;
    const int j = y * nx + x;
    const float q = cq[j];

    if (y <= g.ny - P - 1) {                      // Hx cell
        float acc = 0.0f;
#pragma unroll
        for (int k = 1; k <= P; ++k) acc += coef<P>(k) * (e[j + k * nx] - e[j - (k - 1) * nx]);
        float d = acc * g.rdy;
        if (flag_hy(g, y)) {
            const int64_t m_i = ((int64_t)s * g.by + band_y(g, y)) * nx + x;
            float m = cp[BYH * g.L + y] * psi_ez[m_i] + cp[AYH * g.L + y] * d;
            psi_ez[m_i] = m;
            d = d / cp[KYH * g.L + y] + m;
        }
        Hx[base + j] = Hx[base + j] - q * d;
    }
    if (x <= nx - P - 1) {                        // Hz cell
        float acc = 0.0f;
#pragma unroll
        for (int k = 1; k <= P; ++k) acc += coef<P>(k) * (e[j + k] - e[j - (k - 1)]);
        float d = acc * g.rdx;
        if (flag_hx(g, x)) {
            const int64_t m_i = ((int64_t)s * g.ny + y) * g.bx + band_x(g, x);
            float m = cp[BXH * g.L + x] * psi_ex[m_i] + cp[AXH * g.L + x] * d;
            psi_ex[m_i] = m;
            d = d / cp[KXH * g.L + x] + m;
        }
        Hz[base + j] = Hz[base + j] + q * d;
    }
}

// ---------------------------------------------------------------------------
// Forward E step: Ey = Ca Ey + Cb (filt(Dx Hz) - filt(Dz Hx)), with optional
// snapshot of Ey^n (before the update) and curl H^n on the interior window.
// ---------------------------------------------------------------------------
template <int P, int SNAP>
__global__ __launch_bounds__(BLK_X* BLK_Y) void k_fwd_e(Geo g, const float* __restrict__ ca,
                                                        const float* __restrict__ cb,
                                                        const float* __restrict__ Hx,
                                                        const float* __restrict__ Hz,
                                                        float* __restrict__ E,
                                                        float* __restrict__ psi_hxz,
                                                        float* __restrict__ psi_hzx,
                                                        const float* __restrict__ cp,
                                                        void* __restrict__ snap_e,
                                                        void* __restrict__ snap_c)
{
    const int x = blockIdx.x * BLK_X + threadIdx.x + P;
    const int y = blockIdx.y * BLK_Y + threadIdx.y + P;
    const int s = blockIdx.z;
    if (x > g.nx - P || y > g.ny - P) return;
    const int nx = g.nx;
    const int64_t base = (int64_t)s * g.slab;
    const float* hx = Hx + base;
    const float* hz = Hz + base;
    const int j = y * nx + x;

    float acc = 0.0f;
#pragma unroll
    for (int k = 1; k <= P; ++k) acc += coef<P>(k) * (hz[j + (k - 1)] - hz[j - k]);
    float u = acc * g.rdx;
    if (flag_ex(g, x)) {
        const int64_t m_i = ((int64_t)s * g.ny + y) * g.bx + band_x(g, x);
        float m = cp[BX * g.L + x] * psi_hzx[m_i] + cp[AX * g.L + x] * u;
        psi_hzx[m_i] = m;
        u = u / cp[KX * g.L + x] + m;
    }
    acc = 0.0f;
#pragma unroll
    for (int k = 1; k <= P; ++k) acc += coef<P>(k) * (hx[j + (k - 1) * nx] - hx[j - k * nx]);
    float v = acc * g.rdy;
    if (flag_ey(g, y)) {
        const int64_t m_i = ((int64_t)s * g.by + band_y(g, y)) * nx + x;
        float m = cp[BY * g.L + y] * psi_hxz[m_i] + cp[AY * g.L + y] * v;
        psi_hxz[m_i] = m;
        v = v / cp[KY * g.L + y] + m;
    }
    const float curl = u - v;
    const float ev = E[base + j];
    if constexpr (SNAP != SNAP_NONE) {
        if (y >= g.y0 && y < g.y1 && x >= g.x0 && x < g.x1) {
            const int64_t w = ((int64_t)s * g.nyi + (y - g.y0)) * g.nxi + (x - g.x0);
            snap_store<SNAP>(snap_e, w, ev);
            snap_store<SNAP>(snap_c, w, curl);
        }
    }
    E[base + j] = ca[j] * ev + cb[j] * curl;
}

// ---------------------------------------------------------------------------
// Sources and receivers of one step.  One workgroup per shot: first every
// distinct source cell adds the sum of its sources (ascending source order),
// then, after the barrier, every receiver reads Ey.  Duplicate cells
// therefore never race.
//   cell/ptr/list: per shot, the distinct cells (padded with -1), CSR offsets
//   into list, and list = source indices grouped by cell.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_fwd_srcrec(int64_t slab, float* __restrict__ E,
                                                    const float* __restrict__ f_t, int n_src,
                                                    const int* __restrict__ s_cell,
                                                    const int* __restrict__ s_ptr,
                                                    const int* __restrict__ s_list,
                                                    float* __restrict__ r_t, int n_rec,
                                                    const int* __restrict__ r_idx)
{
    const int s = blockIdx.x;
    float* e = E + (int64_t)s * slab;
    for (int u = threadIdx.x; u < n_src; u += blockDim.x) {
        const int c = s_cell[s * n_src + u];
        if (c < 0) continue;
        const int* ptr = s_ptr + s * (n_src + 1);
        float acc = 0.0f;
        for (int q = ptr[u]; q < ptr[u + 1]; ++q) acc += f_t[s * n_src + s_list[s * n_src + q]];
        e[c] = e[c] + acc;
    }
    __syncthreads();
    if (r_t == nullptr) return;
    for (int i = threadIdx.x; i < n_rec; i += blockDim.x) {
        const int c = r_idx[s * n_rec + i];
        r_t[s * n_rec + i] = c >= 0 ? e[c] : 0.0f;
    }
}

// Adjoint of the above: residuals injected at the receivers (distinct
// receiver cells, ascending receiver order), then the adjoint field read at
// the sources (source-wavelet gradient).
__global__ __launch_bounds__(256) void k_adj_srcrec(int64_t slab, float* __restrict__ lE,
                                                    const float* __restrict__ gr_t, int n_rec,
                                                    const int* __restrict__ r_cell,
                                                    const int* __restrict__ r_ptr,
                                                    const int* __restrict__ r_list,
                                                    float* __restrict__ gf_t, int n_src,
                                                    const int* __restrict__ s_idx)
{
    const int s = blockIdx.x;
    float* e = lE + (int64_t)s * slab;
    for (int u = threadIdx.x; u < n_rec; u += blockDim.x) {
        const int c = r_cell[s * n_rec + u];
        if (c < 0) continue;
        const int* ptr = r_ptr + s * (n_rec + 1);
        float acc = 0.0f;
        for (int q = ptr[u]; q < ptr[u + 1]; ++q) acc += gr_t[s * n_rec + r_list[s * n_rec + q]];
        e[c] = e[c] + acc;
    }
    __syncthreads();
    if (gf_t == nullptr) return;
    for (int i = threadIdx.x; i < n_src; i += blockDim.x) {
        const int c = s_idx[s * n_src + i];
        gf_t[s * n_src + i] = c >= 0 ? e[c] : 0.0f;
    }
}

// ---------------------------------------------------------------------------
// Adjoint band pre-pass over the E cells of the CPML bands.  The linear index
// covers the band rows (all columns) and then the remaining rows' band
// columns, so every band cell is visited once.
// ---------------------------------------------------------------------------
template <int P>
__global__ __launch_bounds__(256) void k_adj_band(Geo g, const float* __restrict__ cb,
                                                  const float* __restrict__ lE,
                                                  float* __restrict__ phi_hzx,
                                                  float* __restrict__ phi_hxz,
                                                  float* __restrict__ Ub, float* __restrict__ Wb,
                                                  const float* __restrict__ cp)
{
    const int s = blockIdx.y;
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    const int part_a = g.by * g.nx;
    int y, x;
    if (idx < part_a) {
        const int yb = idx / g.nx;
        x = idx - yb * g.nx;
        y = yb < g.byl ? yb : g.hy1 + (yb - g.byl);
    } else {
        const int i2 = idx - part_a;
        if (i2 >= (g.ny - g.by) * g.bx) return;
        const int r = i2 / g.bx;
        const int xb = i2 - r * g.bx;
        y = g.y0 + r;
        x = xb < g.bxl ? xb : g.hx1 + (xb - g.bxl);
    }
    const int P_ = g.P;
    if (y < P_ || y > g.ny - P_ || x < P_ || x > g.nx - P_) return;   // not an E cell
    const bool fx = flag_ex(g, x), fy = flag_ey(g, y);
    if (!fx && !fy) return;
    const int j = y * g.nx + x;
    const float h = cb[j] * lE[(int64_t)s * g.slab + j];
    if (fx) {
        const int64_t m_i = ((int64_t)s * g.ny + y) * g.bx + band_x(g, x);
        float m = cp[BX * g.L + x] * phi_hzx[m_i] + cp[AX * g.L + x] * h;
        phi_hzx[m_i] = m;
        Ub[m_i] = h / cp[KX * g.L + x] + m;
    }
    if (fy) {
        const int64_t m_i = ((int64_t)s * g.by + band_y(g, y)) * g.nx + x;
        float m = cp[BY * g.L + y] * phi_hxz[m_i] + cp[AY * g.L + y] * h;
        phi_hxz[m_i] = m;
        Wb[m_i] = h / cp[KY * g.L + y] + m;
    }
}

// ---------------------------------------------------------------------------
// Adjoint lambda_H pass.
// ---------------------------------------------------------------------------
template <int P>
__global__ __launch_bounds__(BLK_X* BLK_Y) void k_adj_h(Geo g, const float* __restrict__ cb,
                                                        const float* __restrict__ cq,
                                                        const float* __restrict__ lE,
                                                        float* __restrict__ lHx,
                                                        float* __restrict__ lHz,
                                                        float* __restrict__ phi_ez,
                                                        float* __restrict__ phi_ex,
                                                        const float* __restrict__ Ub,
                                                        const float* __restrict__ Wb,
                                                        float* __restrict__ TZb,
                                                        float* __restrict__ TXb,
                                                        const float* __restrict__ cp)
{
    const int x = blockIdx.x * BLK_X + threadIdx.x + P;
    const int y = blockIdx.y * BLK_Y + threadIdx.y + P;
    const int s = blockIdx.z;
    if (x > g.nx - P || y > g.ny - P) return;
    const int nx = g.nx;
    const int64_t base = (int64_t)s * g.slab;
    const float* le = lE + base;
    const int j = y * nx + x;
    const int64_t xrow = ((int64_t)s * g.ny + y) * g.bx;      // x-band row of this y

    if (x <= nx - P - 1) {                                    // Hz cell
        auto ubar = [&](int xx) -> float {
            return flag_ex(g, xx) ? Ub[xrow + band_x(g, xx)] : cb[y * nx + xx] * le[y * nx + xx];
        };
        float acc = 0.0f;
#pragma unroll
        for (int k = 1; k <= P; ++k) acc += coef<P>(k) * (ubar(x + k) - ubar(x - k + 1));
        const float lhz = lHz[base + j] - acc * g.rdx;
        lHz[base + j] = lhz;
        if (flag_hx(g, x)) {
            const float qv = cq[j] * lhz;
            const int64_t m_i = xrow + band_x(g, x);
            float m = cp[BXH * g.L + x] * phi_ex[m_i] + cp[AXH * g.L + x] * qv;
            phi_ex[m_i] = m;
            TZb[m_i] = qv / cp[KXH * g.L + x] + m;
        }
    }
    if (y <= g.ny - P - 1) {                                  // Hx cell
        auto wbar = [&](int yy) -> float {
            return flag_ey(g, yy) ? Wb[((int64_t)s * g.by + band_y(g, yy)) * nx + x]
                                  : cb[yy * nx + x] * le[yy * nx + x];
        };
        float acc = 0.0f;
#pragma unroll
        for (int k = 1; k <= P; ++k) acc += coef<P>(k) * (wbar(y + k) - wbar(y - k + 1));
        const float lhx = lHx[base + j] + acc * g.rdy;
        lHx[base + j] = lhx;
        if (flag_hy(g, y)) {
            const float qv = cq[j] * lhx;
            const int64_t m_i = ((int64_t)s * g.by + band_y(g, y)) * nx + x;
            float m = cp[BYH * g.L + y] * phi_ez[m_i] + cp[AYH * g.L + y] * qv;
            phi_ez[m_i] = m;
            TXb[m_i] = qv / cp[KYH * g.L + y] + m;
        }
    }
}

// ---------------------------------------------------------------------------
// Adjoint lambda_E pass with gradient accumulation (interior window only).
// ---------------------------------------------------------------------------
template <int P, int SNAP>
__global__ __launch_bounds__(BLK_X* BLK_Y) void k_adj_e(Geo g, const float* __restrict__ ca,
                                                        const float* __restrict__ cq,
                                                        const float* __restrict__ lHx,
                                                        const float* __restrict__ lHz,
                                                        float* __restrict__ lE,
                                                        const float* __restrict__ TZb,
                                                        const float* __restrict__ TXb,
                                                        const void* __restrict__ snap_e,
                                                        const void* __restrict__ snap_c,
                                                        float* __restrict__ gca,
                                                        float* __restrict__ gcb)
{
    const int x = blockIdx.x * BLK_X + threadIdx.x + P;
    const int y = blockIdx.y * BLK_Y + threadIdx.y + P;
    const int s = blockIdx.z;
    if (x > g.nx - P || y > g.ny - P) return;
    const int nx = g.nx;
    const int64_t base = (int64_t)s * g.slab;
    const int j = y * nx + x;
    const float e = lE[base + j];

    if constexpr (SNAP != SNAP_NONE) {
        if (y >= g.y0 && y < g.y1 && x >= g.x0 && x < g.x1) {
            const int64_t w = ((int64_t)s * g.nyi + (y - g.y0)) * g.nxi + (x - g.x0);
            if (gca) gca[base + j] = gca[base + j] + e * snap_load<SNAP>(snap_e, w);
            if (gcb) gcb[base + j] = gcb[base + j] + e * snap_load<SNAP>(snap_c, w);
        }
    }

    const float* lhz = lHz + base;
    const float* lhx = lHx + base;
    const int64_t xrow = ((int64_t)s * g.ny + y) * g.bx;
    auto tz = [&](int xx) -> float {
        return flag_hx(g, xx) ? TZb[xrow + band_x(g, xx)] : cq[y * nx + xx] * lhz[y * nx + xx];
    };
    auto tx = [&](int yy) -> float {
        return flag_hy(g, yy) ? TXb[((int64_t)s * g.by + band_y(g, yy)) * nx + x]
                              : cq[yy * nx + x] * lhx[yy * nx + x];
    };
    float az = 0.0f, ay = 0.0f;
#pragma unroll
    for (int k = 1; k <= P; ++k) az += coef<P>(k) * (tz(x + k - 1) - tz(x - k));
#pragma unroll
    for (int k = 1; k <= P; ++k) ay += coef<P>(k) * (tx(y + k - 1) - tx(y - k));
    lE[base + j] = ca[j] * e + (-(az * g.rdx) + ay * g.rdy);
}

// ---------------------------------------------------------------------------
// Shot sum (combine_grad): grad[j] = sum_s grad_shot[s][j], ascending s.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_shot_sum(int64_t slab, int n_shots,
                                                  const float* __restrict__ gs,
                                                  float* __restrict__ out)
{
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= slab) return;
    float acc = 0.0f;
    for (int s = 0; s < n_shots; ++s) acc += gs[(int64_t)s * slab + j];
    out[j] = acc;
}

// Fill with zeros (used instead of memset so callers may capture the calls).
__global__ __launch_bounds__(256) void k_zero(float* __restrict__ p, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0.0f;
}

// Max of cb*cq over [0, n): per-block maxima into part[blockIdx.x].
__global__ __launch_bounds__(256) void k_max_cbcq(const float* __restrict__ cb,
                                                  const float* __restrict__ cq, int64_t n,
                                                  float* __restrict__ part)
{
    __shared__ float red[256];
    float m = 0.0f;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const float v = cb[i] * cq[i];
        m = (v > m || v != v) ? v : m;     // NaN propagates
    }
    red[threadIdx.x] = m;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (threadIdx.x < w) {
            const float o = red[threadIdx.x + w];
            red[threadIdx.x] = (o > red[threadIdx.x] || o != o) ? o : red[threadIdx.x];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

}  // namespace tmf
