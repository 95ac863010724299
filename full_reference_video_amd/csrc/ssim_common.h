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

// Raw samples as loaded, and their value on the 8-bit scale.  Loads and
// conversions are separate so that a tile's loads can all be in flight
// before the first conversion waits for one.
__device__ __forceinline__ float to_value(float v, float) { return v; }
__device__ __forceinline__ float to_value(uint8_t v, float unit) { return (float)v * unit; }
__device__ __forceinline__ float to_value(uint16_t v, float unit) { return (float)v * unit; }

// Sum over the 64 lanes of a wave in a fixed butterfly order; every lane
// ends with the same bits.
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// LDS row pitch (floats) of a staged input tile: a multiple of 4 with room
// for the 16-byte reads of the horizontal pass.
template <int TW>
constexpr int in_pitch() {
    static_assert(TW % 4 == 0, "tile width must be a multiple of 4");
    return TW + 12;
}

// LDS of a tile: the staged input (two planes, IH rows of pitch
// in_pitch<TW>()) and, after the horizontal pass, the five horizontal moment
// planes (IH x TW each) in the same buffer.
template <int TW, int TH>
constexpr int tile_lds_floats() {
    constexpr int stage = 2 * (TH + 10) * in_pitch<TW>(), moments = 5 * (TH + 10) * TW;
    return stage > moments ? stage : moments;
}

// LDS float offset, relative to the first staged plane, where threads past a
// staged tile's last cell put their (unused) value, so that every thread
// stores: a store under a per-lane condition lets the compiler sink the
// matching load behind the stores of earlier cells, and the tile then costs
// two memory latencies.  It lies past both staged planes and inside the
// tile's buffer (sized for the moment planes), four floats wide.
template <int TW, int TH>
constexpr int stage_spare() {
    constexpr int IH = TH + 10, IP = in_pitch<TW>();
    static_assert(2 * IH * IP + IH * IP + 4 <= tile_lds_floats<TW, TH>(), "no spare LDS past the staged tile");
    return 2 * IH * IP;
}

// Stage the (TH + 10) x (TW + 10) input tile of both planes at (x0, y0),
// offset-subtracted, in LDS with row pitch in_pitch<TW>().  A cell outside
// the plane (column >= W or row >= H) is read from the plane's first sample
// instead and left as it comes: such cells feed only the moments of map
// pixels outside the valid region, which are never summed, and never the
// next pyramid level (its 2x2 blocks lie inside the plane), so they need an
// in-bounds address but no masking.  Every load is unconditional and all of
// them are issued before the first conversion, so the tile costs one memory
// latency.  (A load under a per-lane branch makes the compiler wait for
// every earlier load before it.)  The conversion raw * unit - 128 is one
// fused multiply-add: raw * unit is exact (unit is a power of two), so it
// rounds once either way.
template <int TW, int TH, int NT, typename TIn>
__device__ __forceinline__ void stage_tile(const TIn *__restrict__ ref, const TIn *__restrict__ dis,
                                           int pitch, int W, int H, float unit, int x0, int y0,
                                           float *sx, float *sy) {
    constexpr int IW = TW + 10, IH = TH + 10, IP = in_pitch<TW>();
    constexpr int N = (IH * IW + NT - 1) / NT;
    TIn ra[N], rb[N];
    int lds_off[N];
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const int i = threadIdx.x + k * NT;
        const int r = i / IW, c = i - r * IW;
        const int gx = x0 + c, gy = y0 + r;
        const bool in = i < IH * IW && gx < W && gy < H;
        const size_t o = in ? (size_t)gy * (size_t)pitch + (size_t)gx : 0;
        ra[k] = ref[o];
        rb[k] = dis[o];
        lds_off[k] = i < IH * IW ? r * IP + c : stage_spare<TW, TH>();
    }
#pragma unroll
    for (int k = 0; k < N; ++k) {
        sx[lds_off[k]] = fmaf(to_value(ra[k], 1.0f), unit, -kMomentOffset);
        sy[lds_off[k]] = fmaf(to_value(rb[k], 1.0f), unit, -kMomentOffset);
    }
}

// Four consecutive raw samples (aligned to 4 samples) as one load, and
// their values on the 8-bit scale with the mid-scale offset removed.
template <typename TIn> struct Raw4;
template <> struct Raw4<float> {
    using type = float4;
    __device__ static float4 load(const float *p) { return *reinterpret_cast<const float4 *>(p); }
    __device__ static float4 centred(float4 v, float) {
        return make_float4(v.x - kMomentOffset, v.y - kMomentOffset, v.z - kMomentOffset, v.w - kMomentOffset);
    }
};
template <> struct Raw4<uint8_t> {
    using type = uint32_t;
    __device__ static uint32_t load(const uint8_t *p) { return *reinterpret_cast<const uint32_t *>(p); }
    __device__ static float4 centred(uint32_t v, float unit) {
        return make_float4(fmaf((float)(v & 0xffu), unit, -kMomentOffset),
                           fmaf((float)((v >> 8) & 0xffu), unit, -kMomentOffset),
                           fmaf((float)((v >> 16) & 0xffu), unit, -kMomentOffset),
                           fmaf((float)(v >> 24), unit, -kMomentOffset));
    }
};
template <> struct Raw4<uint16_t> {
    using type = uint2;
    __device__ static uint2 load(const uint16_t *p) { return *reinterpret_cast<const uint2 *>(p); }
    __device__ static float4 centred(uint2 v, float unit) {
        return make_float4(fmaf((float)(v.x & 0xffffu), unit, -kMomentOffset),
                           fmaf((float)(v.x >> 16), unit, -kMomentOffset),
                           fmaf((float)(v.y & 0xffffu), unit, -kMomentOffset),
                           fmaf((float)(v.y >> 16), unit, -kMomentOffset));
    }
};

// The same with 4-sample loads, for planes whose base is aligned to 4
// samples and whose row pitch is a multiple of 4 samples (x0, a multiple of
// TW, is a multiple of 4).  A chunk that starts inside a row lies wholly
// inside the row's pitch, so it is read whole; a chunk that starts outside
// the plane reads the plane's first chunk instead.  As above, cells outside
// the plane are left unmasked.
template <int TW, int TH, int NT, typename TIn>
__device__ __forceinline__ void stage_tile_x4(const TIn *__restrict__ ref, const TIn *__restrict__ dis, int pitch,
                                              int W, int H, float unit, int x0, int y0, float *sx, float *sy) {
    constexpr int IW = TW + 10, IH = TH + 10, IP = in_pitch<TW>();
    constexpr int QI = (IW + 3) / 4;  // 4-wide chunks per row (the last one partly past the tile)
    constexpr int N = (IH * QI + NT - 1) / NT;
    using R4 = Raw4<TIn>;
    typename R4::type ra[N], rb[N];
    int lds_off[N];
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const int i = threadIdx.x + k * NT;
        const int r = i / QI, q = i - r * QI;
        const int gx = x0 + 4 * q, gy = y0 + r;
        const bool in = i < IH * QI && gx < W && gy < H;
        const size_t o = in ? (size_t)gy * (size_t)pitch + (size_t)gx : 0;
        ra[k] = R4::load(ref + o);
        rb[k] = R4::load(dis + o);
        lds_off[k] = i < IH * QI ? r * IP + 4 * q : stage_spare<TW, TH>();
    }
#pragma unroll
    for (int k = 0; k < N; ++k) {
        *reinterpret_cast<float4 *>(sx + lds_off[k]) = R4::centred(ra[k], unit);
        *reinterpret_cast<float4 *>(sy + lds_off[k]) = R4::centred(rb[k], unit);
    }
}

// Stage with 4-sample loads when `vec4` says the planes allow it (fp32
// planes always do: their pitch is a multiple of 64 floats), else element by
// element.  `vec4` is uniform over the grid.
template <int TW, int TH, int NT, typename TIn>
__device__ __forceinline__ void stage(const TIn *__restrict__ ref, const TIn *__restrict__ dis, int pitch, int W,
                                      int H, float unit, int x0, int y0, float *sx, float *sy, bool vec4) {
    if (vec4)
        stage_tile_x4<TW, TH, NT>(ref, dis, pitch, W, H, unit, x0, y0, sx, sy);
    else
        stage_tile<TW, TH, NT>(ref, dis, pitch, W, H, unit, x0, y0, sx, sy);
}

// Whether planes at this address with this pitch (in samples) can be staged
// with 4-sample loads.
inline bool stage_vec4_ok(const void *p, int pitch, size_t sample_bytes) {
    return ((uintptr_t)p % (4 * sample_bytes)) == 0 && pitch % 4 == 0;
}

// Hardware reciprocal and square root (v_rcp_f32, v_sqrt_f32: about 1 ulp).
// The map terms are written so that identical planes stay exactly 1 anyway.
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float hw_sqrt(float x) { return __builtin_amdgcn_sqrtf(x); }

// Per-pixel SSIM term from the five (offset) moments, as
// (1 - (mx - my)^2 / A)(1 - v / B) with A = mux^2 + muy^2 + C1,
// B = sxx + syy + C2 and v = sxx + syy - 2 sxy (the variance of x - y):
// algebraically ((2 mux muy + C1)(2 sxy + C2)) / (A B), and exactly 1 for
// identical planes, since then mx = my and sxx = syy = sxy bit for bit.
__device__ __forceinline__ float ssim_term(float mx, float my, float xx, float yy, float xy) {
    const float sxx = xx - mx * mx;
    const float syy = yy - my * my;
    const float sxy = xy - mx * my;
    const float ux = mx + kMomentOffset;
    const float uy = my + kMomentOffset;
    const float dm = mx - my;
    const float A = ux * ux + uy * uy + kC1;
    const float B = sxx + syy + kC2;
    const float v = (sxx + syy) - (sxy + sxy);
    // One reciprocal for both quotients (A * B stays far inside fp32 range).
    const float r = rcp(A * B);
    return (1.0f - dm * dm * (B * r)) * (1.0f - v * (A * r));
}

// Horizontal 11-tap pass of one item: four adjacent columns c0..c0+3 of
// tile row r, for x, y, x^2, y^2 and xy, from the 14 inputs of each plane
// (FMA order k = 0..10).
__device__ __forceinline__ void h_item_load(const float *pa, const float *pb, float (&a)[14], float (&b)[14]) {
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        const float4 va = *reinterpret_cast<const float4 *>(pa + 4 * q);
        const float4 vb = *reinterpret_cast<const float4 *>(pb + 4 * q);
        a[4 * q] = va.x; a[4 * q + 1] = va.y; a[4 * q + 2] = va.z; a[4 * q + 3] = va.w;
        b[4 * q] = vb.x; b[4 * q + 1] = vb.y; b[4 * q + 2] = vb.z; b[4 * q + 3] = vb.w;
    }
    const float2 va = *reinterpret_cast<const float2 *>(pa + 12);
    const float2 vb = *reinterpret_cast<const float2 *>(pb + 12);
    a[12] = va.x; a[13] = va.y;
    b[12] = vb.x; b[13] = vb.y;
}

__device__ __forceinline__ void h_item_compute(const float (&a)[14], const float (&b)[14], const Taps &taps,
                                               float (&m)[5][4]) {
    float aa[14], bb[14], ab[14];
#pragma unroll
    for (int i = 0; i < 14; ++i) {
        aa[i] = a[i] * a[i];
        bb[i] = b[i] * b[i];
        ab[i] = a[i] * b[i];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) m[0][j] = m[1][j] = m[2][j] = m[3][j] = m[4][j] = 0.f;
#pragma unroll
    for (int k = 0; k < 11; ++k) {
        const float g = taps.g[k];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            m[0][j] = fmaf(g, a[j + k], m[0][j]);
            m[1][j] = fmaf(g, b[j + k], m[1][j]);
            m[2][j] = fmaf(g, aa[j + k], m[2][j]);
            m[3][j] = fmaf(g, bb[j + k], m[3][j]);
            m[4][j] = fmaf(g, ab[j + k], m[4][j]);
        }
    }
}

// The horizontal pass over a staged tile, in place: the moment planes
// (plane p at lds + p * IH * TW, row pitch TW) overwrite the staged input.
// Each thread has at most two items (row, four columns).  It computes its
// first item and reads the inputs of its second into registers, then the
// workgroup synchronises, and only then are the moments written — so the
// tile needs the LDS of the larger of the two layouts, not of both, and more
// workgroups fit on a CU.  Ends with the moment planes visible to the whole
// workgroup.
template <int TW, int TH, int NT>
__device__ __forceinline__ void horizontal_moments_in_place(float *lds, const Taps &taps) {
    constexpr int IH = TH + 10, IP = in_pitch<TW>(), QW = TW / 4, PL = IH * TW;
    constexpr int ITEMS = IH * QW;
    static_assert(ITEMS <= 2 * NT, "at most two horizontal items per thread");
    const float *sx = lds, *sy = lds + IH * IP;
    const int i1 = threadIdx.x, i2 = threadIdx.x + NT;
    const bool has1 = i1 < ITEMS, has2 = i2 < ITEMS;
    const int r1 = i1 / QW, c1 = (i1 - r1 * QW) * 4;
    const int r2 = i2 / QW, c2 = (i2 - r2 * QW) * 4;
    float m[5][4];
    float a[14], b[14];
    if (has1) {
        h_item_load(sx + r1 * IP + c1, sy + r1 * IP + c1, a, b);
        h_item_compute(a, b, taps, m);
    }
    if (has2) h_item_load(sx + r2 * IP + c2, sy + r2 * IP + c2, a, b);
    __syncthreads();  // every read of the staged tile is done
    if (has1) {
        const int o = r1 * TW + c1;
#pragma unroll
        for (int p = 0; p < 5; ++p)
            *reinterpret_cast<float4 *>(lds + p * PL + o) = make_float4(m[p][0], m[p][1], m[p][2], m[p][3]);
    }
    if (has2) {
        h_item_compute(a, b, taps, m);
        const int o = r2 * TW + c2;
#pragma unroll
        for (int p = 0; p < 5; ++p)
            *reinterpret_cast<float4 *>(lds + p * PL + o) = make_float4(m[p][0], m[p][1], m[p][2], m[p][3]);
    }
    __syncthreads();
}

// Vertical pass: for RB stacked map rows of one tile column at a time, the
// five moments from RB + 10 values of each horizontal plane (FMA order
// k = 0..10), handed to `fn(r, c, mx, my, xx, yy, xy)` for every map pixel
// inside the valid region (mx0 = x0 + c < MW, y0 + r < MH).
template <int TW, int TH, int NT, int RB, typename F>
__device__ __forceinline__ void vertical_moments(const float *hm, const Taps &taps, int x0, int y0, int MW,
                                                 int MH, F &&fn) {
    static_assert(TH % RB == 0, "tile height must be a multiple of the row block");
    constexpr int IH = TH + 10, PL = IH * TW;
    for (int it = threadIdx.x; it < (TH / RB) * TW; it += NT) {
        const int c = it % TW, r0 = (it / TW) * RB;
        if (x0 + c >= MW || y0 + r0 >= MH) continue;
        float m[5][RB];
#pragma unroll
        for (int p = 0; p < 5; ++p) {
            float v[RB + 10];
#pragma unroll
            for (int i = 0; i < RB + 10; ++i) v[i] = hm[p * PL + (r0 + i) * TW + c];
#pragma unroll
            for (int j = 0; j < RB; ++j) {
                float acc = 0.f;
#pragma unroll
                for (int k = 0; k < 11; ++k) acc = fmaf(taps.g[k], v[j + k], acc);
                m[p][j] = acc;
            }
        }
#pragma unroll
        for (int j = 0; j < RB; ++j)
            if (y0 + r0 + j < MH) fn(r0 + j, c, m[0][j], m[1][j], m[2][j], m[3][j], m[4][j]);
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

// Sum over the 64 lanes of a wave in fp32, in the same fixed butterfly order.
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Workgroup sum of a tile's map terms: each thread's few terms and then the
// wave's 64 lanes are summed in fp32 (a wave holds a few hundred terms, each
// of magnitude at most 1, so the fp32 sum is good to about 1e-5 of a term),
// the waves in index order in fp64.  Fixed shape; `out` is valid in thread 0
// only and `red` may be reused after the next __syncthreads.
template <int NT, int NV>
__device__ __forceinline__ void block_sum_terms(const float (&v)[NV], double (*red)[NT / 64], double (&out)[NV]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const float w = wave_sum_f32(v[j]);
        if (lane == 0) red[j][wave] = (double)w;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            double t = 0.0;
            for (int w = 0; w < NT / 64; ++w) t += red[j][w];
            out[j] = t;
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
    // Eight loads in flight per thread and span; the additions keep the
    // index order (a slot past the span adds +0.0, which changes nothing).
    constexpr int U = 8;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const double *p = partials + (size_t)j * stride;
        double t = 0.0;
        for (int i0 = threadIdx.x; i0 < nb; i0 += U * NT) {
            double v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = i0 + u * NT;
                v[u] = p[i < nb ? i : nb - 1];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) t += i0 + u * NT < nb ? v[u] : 0.0;
        }
        tot[j] = t;
    }
    block_sum<NT, NV>(tot, red);
}

}  // namespace vqm
