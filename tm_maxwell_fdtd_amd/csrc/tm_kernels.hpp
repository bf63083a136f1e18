// Small kernels around the time-step kernels: source injection and
// receiver gather and their adjoints, the gradient shot sum (tide-GPR
// 0.0.9, maxwell.cu: combine_grad), the chain rule to eps_r / sigma
// gradients, a fill kernel and the Courant-number reduction (gfx950,
// wave64).
#pragma once

#include "tm_common.hpp"

namespace tmf {

// ---------------------------------------------------------------------------
// Sources and receivers of one step (tide-GPR 0.0.9, maxwell.cu:
// add_sources_ey, record_receivers_ey), on the Ey of a state set whose
// shots are blocks of shot_bytes with Ey at byte oE.  One workgroup per
// shot: first every
// distinct source cell adds the sum of its sources (ascending source order),
// then, after the barrier, every receiver reads Ey.  Duplicate cells
// therefore never race.
//   cell/ptr/list: per shot, the distinct cells (padded with -1), CSR offsets
//   into list, and list = source indices grouped by cell.
// ---------------------------------------------------------------------------
//   rec_rows/r_gather/r_prev (optional): after a two-step launch, the
//   receivers of the launch's first step are gathered from the receiver-row
//   buffer the step kernel wrote (r_gather = slot * nx + x, or -1).
__global__ __launch_bounds__(256) void k_fwd_srcrec(char* __restrict__ set, uint64_t shot_bytes, uint32_t oE,
                                                    const float* __restrict__ f_t, int n_src,
                                                    const int* __restrict__ s_cell,
                                                    const int* __restrict__ s_ptr,
                                                    const int* __restrict__ s_list,
                                                    float* __restrict__ r_t, int n_rec,
                                                    const int* __restrict__ r_idx,
                                                    const float* __restrict__ rec_rows,
                                                    const int* __restrict__ r_gather,
                                                    float* __restrict__ r_prev, int n_slots, int nx)
{
    const int s = blockIdx.x;
    if (r_prev != nullptr) {
        for (int i = threadIdx.x; i < n_rec; i += blockDim.x) {
            const int gidx = r_gather[s * n_rec + i];
            r_prev[s * n_rec + i] = gidx >= 0 ? rec_rows[(int64_t)s * n_slots * nx + gidx] : 0.0f;
        }
    }
    float* e = reinterpret_cast<float*>(set + (uint64_t)s * shot_bytes + oE);
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

// Adjoint of the above (add_adjoint_sources_ey, record_adjoint_at_sources):
// residuals injected at the receivers (distinct
// receiver cells, ascending receiver order), then the adjoint field read at
// the sources (source-wavelet gradient).
__global__ __launch_bounds__(256) void k_adj_srcrec(char* __restrict__ set, uint64_t shot_bytes, uint32_t oE,
                                                    const float* __restrict__ gr_t, int n_rec,
                                                    const int* __restrict__ r_cell,
                                                    const int* __restrict__ r_ptr,
                                                    const int* __restrict__ r_list,
                                                    float* __restrict__ gf_t, int n_src,
                                                    const int* __restrict__ s_idx)
{
    const int s = blockIdx.x;
    float* e = reinterpret_cast<float*>(set + (uint64_t)s * shot_bytes + oE);
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

// Gradients in the physical parameters (tide-GPR 0.0.9, maxwell.cu:
// convert_grad_ca_cb_to_eps_sigma).  With s = sigma dt / (2 eps) and
// eps = EP0 eps_r, Ca = (1 - s) / (1 + s) and Cb = (dt / eps) / (1 + s), so
//   dCa/deps = (1 - Ca) Cb / dt,  dCb/deps = -Cb^2 / dt,
//   dCa/dsigma = -(1 + Ca) Cb / 2,  dCb/dsigma = -Cb^2 / 2,
// and dJ/deps_r = EP0 (gCa dCa/deps + gCb dCb/deps).  A null gradient input
// counts as zero; a null output is skipped.
// ---------------------------------------------------------------------------
constexpr float EP0 = 8.8541878128e-12f;

__global__ __launch_bounds__(256) void k_eps_sigma(int64_t n, const float* __restrict__ ca,
                                                   const float* __restrict__ cb,
                                                   const float* __restrict__ gca,
                                                   const float* __restrict__ gcb, float inv_dt,
                                                   float* __restrict__ geps, float* __restrict__ gsig)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride) {
        const float a = ca[j], b = cb[j];
        const float ga = gca != nullptr ? gca[j] : 0.0f;
        const float gb = gcb != nullptr ? gcb[j] : 0.0f;
        const float b2 = b * b;
        const float dca_de = (1.0f - a) * b * inv_dt;
        const float dcb_de = -b2 * inv_dt;
        const float dca_ds = -0.5f * (1.0f + a) * b;
        const float dcb_ds = -0.5f * b2;
        if (geps != nullptr) geps[j] = (ga * dca_de + gb * dcb_de) * EP0;
        if (gsig != nullptr) gsig[j] = ga * dca_ds + gb * dcb_ds;
    }
}

// ---------------------------------------------------------------------------
// Element-wise conversion to and from the FP8 E4M3 snapshot encoding
// (f32_to_e4m3 / e4m3_to_f32).
__global__ __launch_bounds__(256) void k_fp8_encode(const float* __restrict__ in, uint8_t* __restrict__ out,
                                                    int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
        out[j] = (uint8_t)f32_to_e4m3(in[j]);
}
__global__ __launch_bounds__(256) void k_fp8_decode(const uint8_t* __restrict__ in, float* __restrict__ out,
                                                    int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
        out[j] = e4m3_to_f32(in[j]);
}

// ---------------------------------------------------------------------------
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
