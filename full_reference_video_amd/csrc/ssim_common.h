// ssim_common.h — device helpers shared by the SSIM-map and MS-SSIM level
// kernels (library-private): tile staging, the separable 11-tap moments, and
// the fixed-shape reductions.
//
// The reduction has two launches: every map workgroup writes its own fixed-
// tree partial to a partials array indexed by its tile, and a finish kernel
// with one workgroup per frame sums the partials in index order ("Research-
// 1363: Device-resident ssimulacra2 and a single-wait MS-SSIM on SYCL",
// Finding 4: a work-group tree, then one group over the partials).  A
// last-workgroup-arrives ticket would save the launch, but on gfx950 each
// device-scope release/acquire around it writes back and invalidates the
// XCD's L2, which costs several times the map itself.
#pragma once

#include "vqm_kernels.h"

namespace vqm {

// SSIM stabilisers on the 8-bit scale (L = 255, K1 = 0.01, K2 = 0.03).
constexpr float kC1 = (float)((0.01 * 255.0) * (0.01 * 255.0));
constexpr float kC2 = (float)((0.03 * 255.0) * (0.03 * 255.0));

template <typename TIn>
__device__ __forceinline__ float load_sample(const TIn *p, size_t i, float unit);
template <>
__device__ __forceinline__ float load_sample<float>(const float *p, size_t i, float) { return p[i]; }
template <>
__device__ __forceinline__ float load_sample<uint8_t>(const uint8_t *p, size_t i, float unit) {
    return (float)p[i] * unit;
}
template <>
__device__ __forceinline__ float load_sample<uint16_t>(const uint16_t *p, size_t i, float unit) {
    return (float)p[i] * unit;
}

// Sum over the 64 lanes of a wave in a fixed butterfly order; every lane
// ends with the same bits.
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Stage the (TH + 10) x (TW + 10) input tile of both planes at (x0, y0),
// offset-subtracted, in LDS; cells outside the plane hold 0 (they feed only
// map pixels outside the valid region).
template <int TW, int TH, int NT, typename TIn>
__device__ __forceinline__ void stage_tile(const TIn *__restrict__ ref, const TIn *__restrict__ dis,
                                           int pitch, int W, int H, float unit, int x0, int y0,
                                           float *sx, float *sy) {
    constexpr int IW = TW + 10, IH = TH + 10;
    for (int i = threadIdx.x; i < IH * IW; i += NT) {
        const int r = i / IW, c = i - r * IW;
        const int gx = x0 + c, gy = y0 + r;
        float a = 0.0f, b = 0.0f;
        if (gx < W && gy < H) {
            const size_t o = (size_t)gy * (size_t)pitch + (size_t)gx;
            a = load_sample(ref, o, unit) - kMomentOffset;
            b = load_sample(dis, o, unit) - kMomentOffset;
        }
        sx[i] = a;
        sy[i] = b;
    }
}

// Horizontal pass: the five Gaussian moments of every staged row at each of
// the TW map columns, into five LDS planes of (TH + 10) x TW.
template <int TW, int TH, int NT>
__device__ __forceinline__ void horizontal_moments(const float *sx, const float *sy, const Taps &taps,
                                                   float *hmx, float *hmy, float *hxx, float *hyy,
                                                   float *hxy) {
    constexpr int IW = TW + 10, IH = TH + 10;
    for (int i = threadIdx.x; i < IH * TW; i += NT) {
        const int r = i / TW, c = i - r * TW;
        const float *px = sx + r * IW + c;
        const float *py = sy + r * IW + c;
        float mx = 0.f, my = 0.f, xx = 0.f, yy = 0.f, xy = 0.f;
#pragma unroll
        for (int k = 0; k < 11; ++k) {
            const float a = px[k], b = py[k], g = taps.g[k];
            mx = fmaf(g, a, mx);
            my = fmaf(g, b, my);
            xx = fmaf(g, a * a, xx);
            yy = fmaf(g, b * b, yy);
            xy = fmaf(g, a * b, xy);
        }
        hmx[i] = mx;
        hmy[i] = my;
        hxx[i] = xx;
        hyy[i] = yy;
        hxy[i] = xy;
    }
}

// Vertical pass at map pixel (r, c) of the tile: the five moments.
template <int TW>
__device__ __forceinline__ void vertical_moments(const float *hmx, const float *hmy, const float *hxx,
                                                 const float *hyy, const float *hxy, const Taps &taps,
                                                 int r, int c, float &mx, float &my, float &xx,
                                                 float &yy, float &xy) {
    mx = my = xx = yy = xy = 0.f;
#pragma unroll
    for (int k = 0; k < 11; ++k) {
        const int o = (r + k) * TW + c;
        const float g = taps.g[k];
        mx = fmaf(g, hmx[o], mx);
        my = fmaf(g, hmy[o], my);
        xx = fmaf(g, hxx[o], xx);
        yy = fmaf(g, hyy[o], yy);
        xy = fmaf(g, hxy[o], xy);
    }
}

// Workgroup sum of NV doubles per thread in a fixed shape: wave butterflies,
// then the waves in index order.  Valid in thread 0 only.  `red` may be
// reused after the next __syncthreads.
template <int NT, int NV>
__device__ __forceinline__ void block_sum(double (&v)[NV], double (*red)[NT / 64]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        v[j] = wave_sum(v[j]);
        if (lane == 0) red[j][wave] = v[j];
    }
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            double t = 0.0;
            for (int w = 0; w < NT / 64; ++w) t += red[j][w];
            v[j] = t;
        }
    }
}

// In a one-workgroup-per-frame finish kernel: sum each of NV spans of `nb`
// partials (span j at partials + j * stride) in a fixed shape — thread t
// takes partials t, t + NT, ... in index order, then block_sum.  The
// partials were written by an earlier kernel on the same stream, so the
// kernel boundary has made them visible.  Thread 0 holds the totals.
template <int NT, int NV>
__device__ __forceinline__ void sum_spans(const double *partials, int nb, size_t stride, double (&tot)[NV],
                                          double (*red)[NT / 64]) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        double t = 0.0;
        for (int i = threadIdx.x; i < nb; i += NT) t += partials[(size_t)j * stride + i];
        tot[j] = t;
    }
    block_sum<NT, NV>(tot, red);
}

}  // namespace vqm
