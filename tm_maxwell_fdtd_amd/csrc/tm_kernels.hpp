// Small kernels around the time-step kernels: the event rows of the
// sources and receivers, the gradient shot sum (tide-GPR
// 0.0.9, maxwell.cu: combine_grad), the chain rule to eps_r / sigma
// gradients, a fill kernel and the Courant-number reduction (gfx950,
// wave64).
#pragma once

#include "tm_common.hpp"

namespace tmf {

// ---------------------------------------------------------------------------
// Event rows of a run of steps (tide-GPR 0.0.9, maxwell.cu: add_sources_ey
// and record_receivers_ey, and their adjoints).  Slot g is one grid row of
// shot slot_shot[g] that holds sources or receivers; colcell[g][x] is the
// cell number of (that row, x), or -1.
//
// k_event_add: rows[j][g][x] = the sum of in[j][s][list[q]] over the cell's
// entries q = ptr[k] .. ptr[k+1]-1 (in list order, ascending index), 0 at
// cells without entries; j = 0 .. n_steps-1, in = the first step's values
// [n_steps][S][n_in] (null when n_in = 0: rows of zeros).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_event_add(float* __restrict__ rows, int64_t n, int n_slots, int nx,
                                                   const int* __restrict__ colcell,
                                                   const int* __restrict__ slot_shot,
                                                   const int* __restrict__ ptr, const int* __restrict__ list,
                                                   const float* __restrict__ in, int S, int n_in)
{
    const int64_t row = (int64_t)n_slots * nx;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t j = i / row;
        const int gx = (int)(i - j * row);
        const int k = colcell[gx];
        float acc = 0.0f;
        if (k >= 0 && in != nullptr) {
            const float* v = in + (j * S + slot_shot[gx / nx]) * n_in;
            for (int q = ptr[k]; q < ptr[k + 1]; ++q) acc += v[list[q]];
        }
        rows[i] = acc;
    }
}

// k_event_gather: out[j][i] = rows[j][pos[i]] for the S*n_out entries i of
// each step (pos = g*nx + x of the entry's cell, or -1: absent, 0).
__global__ __launch_bounds__(256) void k_event_gather(float* __restrict__ out, int64_t n, int per_step,
                                                      const int* __restrict__ pos,
                                                      const float* __restrict__ rows, int64_t row_step)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t j = i / per_step;
        const int p = pos[i - j * per_step];
        out[i] = p >= 0 ? rows[j * row_step + p] : 0.0f;
    }
}

// ---------------------------------------------------------------------------
// Shot sum (combine_grad): grad[j] = sum_s grad_shot[s][j], ascending s.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_shot_sum(int64_t slab, int n_shots,
                                                  const float* __restrict__ gs0, float* __restrict__ out0,
                                                  const float* __restrict__ gs1, float* __restrict__ out1)
{
    // blockIdx.y picks the pair (the Ca and the Cb gradients in one launch)
    const float* __restrict__ gs = blockIdx.y ? gs1 : gs0;
    float* __restrict__ out = blockIdx.y ? out1 : out0;
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

// The scan of the Courant check over [0, n), one pass: block b writes the
// largest cb*cq it saw into part[b] (a NaN wins), and into part[nb + b]
// 1.0f if any cq value it saw differs in its bits from q[0], else 0.0f;
// block 0 also writes q[0]'s bits into part[2 nb].
__global__ __launch_bounds__(256) void k_courant_scan(const float* __restrict__ cb,
                                                      const float* __restrict__ cq, int64_t n,
                                                      float* __restrict__ part)
{
    __shared__ float red[256];
    __shared__ int diff_any;
    if (threadIdx.x == 0) diff_any = 0;
    __syncthreads();
    const uint32_t ref = __float_as_uint(cq[0]);
    float m = 0.0f;
    bool diff = false;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const float q = cq[i];
        const float v = cb[i] * q;
        m = (v > m || v != v) ? v : m;     // NaN propagates
        diff |= __float_as_uint(q) != ref;
    }
    if (diff) diff_any = 1;                // every writer stores the same value
    red[threadIdx.x] = m;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (threadIdx.x < w) {
            const float o = red[threadIdx.x + w];
            red[threadIdx.x] = (o > red[threadIdx.x] || o != o) ? o : red[threadIdx.x];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        part[blockIdx.x] = red[0];
        part[gridDim.x + blockIdx.x] = diff_any ? 1.0f : 0.0f;
        if (blockIdx.x == 0) part[2 * gridDim.x] = __uint_as_float(ref);
    }
}

// Up to FILL_JOBS copies and zero fills in one launch: job j (blockIdx.y)
// copies n[j] floats from src[j] to dst[j], or writes n[j] zeros where
// src[j] is null.
constexpr int FILL_JOBS = 8;
struct FillJobs {
    float* dst[FILL_JOBS];
    const float* src[FILL_JOBS];
    int64_t n[FILL_JOBS];
};

__global__ __launch_bounds__(256) void k_fill(FillJobs jobs)
{
    const int j = blockIdx.y;
    float* __restrict__ d = jobs.dst[j];
    const float* __restrict__ s = jobs.src[j];
    const int64_t n = jobs.n[j];
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    if (s != nullptr) {
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) d[i] = s[i];
    } else {
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) d[i] = 0.0f;
    }
}

}  // namespace tmf
