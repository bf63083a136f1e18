// Shared device-side definitions of the TM FDTD kernels (gfx950, wave64).
//
// Notation follows tide-GPR 0.0.9 tide/csrc/maxwell.cu: fields Ey, Hx, Hz;
// update coefficients Ca, Cb (E) and Cq (H); CPML arrays a, b, kappa on the
// integer grid (E-update derivatives) and on the half grid (H-update
// derivatives); FD_PAD = P = order / 2 zero halo cells per side.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tmf {

// Geometry handed to every kernel by value.
struct Geo {
    int ny, nx, P;
    int y0, y1, x0, x1;   // interior window [y0, y1) x [x0, x1)
    int hy1, hx1;         // upper bound of the H-flag interior: y1 - 1, x1 - 1
    int byl, by;          // band rows: [0, y0) -> [0, byl), [y1-1, ny) -> byl + (y - (y1-1))
    int bxl, bx;          // band columns, same mapping along x
    int nyi, nxi;         // interior window size (snapshot slab)
    int L;                // row length of the packed CPML table
    float rdy, rdx;       // 1/dy, 1/dx
    int64_t slab;         // ny * nx
};

// Rows of the packed CPML table [12][L].
enum CpmlRow { AY = 0, BY, KY, AYH, BYH, KYH, AX, BX, KX, AXH, BXH, KXH };

// Staggered-grid Taylor coefficients c_1..c_P (the page's stencil header is
// not on the page; these are the standard staggered coefficients).
template <int P>
__device__ __forceinline__ constexpr float coef(int k);

template <>
__device__ __forceinline__ constexpr float coef<1>(int) { return 1.0f; }
template <>
__device__ __forceinline__ constexpr float coef<2>(int k)
{
    return k == 1 ? (float)(9.0 / 8.0) : (float)(-1.0 / 24.0);
}
template <>
__device__ __forceinline__ constexpr float coef<4>(int k)
{
    return k == 1 ? (float)(1225.0 / 1024.0)
         : k == 2 ? (float)(-245.0 / 3072.0)
         : k == 3 ? (float)(49.0 / 5120.0)
                  : (float)(-5.0 / 7168.0);
}

// Wait until every vector memory access this wave has issued is done
// (vmcnt 0, the other counters left alone).  Resident kernels call it once
// before their time loop: a value loaded before the loop and carried
// through it otherwise looks possibly in flight at the loop head, and the
// compiler then places a wait on it inside the loop, which at every step
// also waits for that step's prefetches and snapshot stores.
__device__ __forceinline__ void drain_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ int band_x(const Geo& g, int x) { return x < g.x0 ? x : g.bxl + (x - g.hx1); }
__device__ __forceinline__ int band_y(const Geo& g, int y) { return y < g.y0 ? y : g.byl + (y - g.hy1); }

// CPML flags: E derivatives outside [lo, hi), H derivatives outside [lo, hi-1).
__device__ __forceinline__ bool flag_ex(const Geo& g, int x) { return x < g.x0 || x >= g.x1; }
__device__ __forceinline__ bool flag_ey(const Geo& g, int y) { return y < g.y0 || y >= g.y1; }
__device__ __forceinline__ bool flag_hx(const Geo& g, int x) { return x < g.x0 || x >= g.hx1; }
__device__ __forceinline__ bool flag_hy(const Geo& g, int y) { return y < g.y0 || y >= g.hy1; }

// float -> bfloat16 bits, round to nearest even (NaN kept quiet).
// Written as a select, not a branch, so it adds no exec-mask changes to the
// step kernels' row loops.
__device__ __forceinline__ uint16_t f32_to_bf16(float v)
{
    const uint32_t u = __float_as_uint(v);
    const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    const uint32_t quiet = (u >> 16) | 0x40u;
    return (uint16_t)(((u & 0x7fffffffu) > 0x7f800000u) ? quiet : rounded);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> OCP FP8 E4M3 bits (the E4M3FN encoding: exponent bias 7, no
// infinities, largest finite 448), round to nearest even; finite values
// beyond +-448 saturate to +-448 and NaN stays NaN.  The conversion
// instruction rounds; the input is clamped first so that no finite value
// becomes NaN.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v)
{
    const float c = __builtin_isnan(v) ? v : fminf(fmaxf(v, -448.0f), 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, 0.0f, 0, false) & 0xffu;
}
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) { return __builtin_amdgcn_cvt_f32_fp8((int)b, 0); }

// Snapshot element types.
enum SnapKind { SNAP_NONE = 0, SNAP_F32 = 1, SNAP_BF16 = 2, SNAP_FP8 = 3 };

// Bytes of one snapshot element.
template <int SNAP>
constexpr uint32_t snap_bytes() { return SNAP == SNAP_BF16 ? 2u : SNAP == SNAP_FP8 ? 1u : 4u; }

}  // namespace tmf
