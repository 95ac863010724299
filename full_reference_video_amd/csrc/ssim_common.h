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

// The separable pass filters NP moment planes.  float_ssim needs the two
// variances only as their sum, so it filters four: x, y, x^2 + y^2 and xy.
// MS-SSIM's contrast term needs sigma_x and sigma_y apart, so it filters
// five: x, y, x^2, y^2 and xy.
template <int NP>
constexpr bool valid_moment_set() {
    return NP == 4 || NP == 5;
}

// LDS float offset, relative to the first staged plane, where threads past a
// staged tile's last cell put their (unused) value, so that every thread
// stores: a store under a per-lane condition lets the compiler sink the
// matching load behind the stores of earlier cells, and the tile then costs
// two memory latencies.  It lies past both staged planes, four floats wide
// (for either plane's base, so up to 3 IH IP + 4 floats into the buffer).
template <int TW, int TH>
constexpr int stage_spare() {
    return 2 * (TH + 10) * in_pitch<TW>();
}

// LDS of a tile: the staged input (two planes, IH rows of pitch
// in_pitch<TW>(), plus the spare slot) and, after the horizontal pass, the NP
// horizontal moment planes (IH x TW each) in the same buffer.
template <int TW, int TH, int NP>
constexpr int tile_lds_floats() {
    static_assert(valid_moment_set<NP>(), "four or five moment planes");
    constexpr int stage = 3 * (TH + 10) * in_pitch<TW>() + 4, moments = NP * (TH + 10) * TW;
    return stage > moments ? stage : moments;
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

// The sum of two squares as the four-plane set forms it: fma(a, a, b * b).
// When a = b this is 2 fl(a^2) exactly: the exact a^2 + fl(a^2) lies within a
// quarter of an ulp of 2 fl(a^2).
__device__ __forceinline__ float sum_of_squares(float a, float b) { return fmaf(a, a, b * b); }

// Per-pixel SSIM term from the four (offset) moments mx, my, ss = E[x^2 + y^2]
// and xy = E[xy], as (1 - (mx - my)^2 / A)(1 - v / B) with
// A = mux^2 + muy^2 + C1, S = sxx + syy = ss - (mx^2 + my^2), B = S + C2 and
// v = S - 2 sxy (the variance of x - y): algebraically
// ((2 mux muy + C1)(2 sxy + C2)) / (A B).  Exactly 1 for identical planes:
// then every x^2 + y^2 is 2 fl(x^2), and doubling commutes with each rounding
// of the filters, so ss = 2 xy, mx = my and S = 2 sxy bit for bit.
// Written with explicit fused multiply-adds (the library compiles with
// contraction off): about 21 instructions.  Identity still gives exactly 1:
// dm = 0, and v = S - 2 sxy is one rounding of an exact 0 (sxy rounds mx my
// first, as S rounds its squares, so S = 2 sxy bit for bit).
__device__ __forceinline__ float ssim_term4(float mx, float my, float ss, float xy) {
    const float S = ss - sum_of_squares(mx, my);
    const float sxy = xy - mx * my;
    const float ux = mx + kMomentOffset;
    const float uy = my + kMomentOffset;
    const float dm = mx - my;
    const float A = fmaf(ux, ux, fmaf(uy, uy, kC1));
    const float B = S + kC2;
    const float v = fmaf(-2.0f, sxy, S);
    // One reciprocal for both quotients (A * B stays far inside fp32 range).
    const float r = rcp(A * B);
    return fmaf(-(dm * dm), B * r, 1.0f) * fmaf(-v, A * r, 1.0f);
}

// Horizontal 11-tap pass of one item: four adjacent columns c0..c0+3 of
// tile row r, for the NP moment planes, from the 14 inputs of each plane
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

template <int NP>
__device__ __forceinline__ void h_item_compute(const float (&a)[14], const float (&b)[14], const Taps &taps,
                                               float (&m)[NP][4]) {
    static_assert(valid_moment_set<NP>(), "four or five moment planes");
    float q[NP - 2][14];  // the second-order products of each input
#pragma unroll
    for (int i = 0; i < 14; ++i) {
        if constexpr (NP == 5) {
            q[0][i] = a[i] * a[i];
            q[1][i] = b[i] * b[i];
            q[2][i] = a[i] * b[i];
        } else {
            q[0][i] = sum_of_squares(a[i], b[i]);
            q[1][i] = a[i] * b[i];
        }
    }
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int j = 0; j < 4; ++j) m[p][j] = 0.f;
#pragma unroll
    for (int k = 0; k < 11; ++k) {
        const float g = taps.g[k];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            m[0][j] = fmaf(g, a[j + k], m[0][j]);
            m[1][j] = fmaf(g, b[j + k], m[1][j]);
#pragma unroll
            for (int p = 0; p < NP - 2; ++p) m[2 + p][j] = fmaf(g, q[p][j + k], m[2 + p][j]);
        }
    }
}

// The horizontal pass over a staged tile, in place: the moment planes
// (plane p at lds + p * IH * TW, row pitch TW) overwrite the staged input.
// Item i is row i / (TW/4), columns 4 (i % (TW/4)) on.  (Reading two staged
// rows whose offsets differ by half the LDS banks in one step instead halves
// the bank conflicts, 18 % -> 10 % of LDS-active cycles, but the kernels are
// VALU-bound and ran no faster.)
// Each thread has at most two items (row, four columns).  It computes its
// first item and reads the inputs of its second into registers, then the
// workgroup synchronises, and only then are the moments written — so the
// tile needs the LDS of the larger of the two layouts, not of both, and more
// workgroups fit on a CU.  Ends with the moment planes visible to the whole
// workgroup.
template <int TW, int TH, int NT, int NP>
__device__ __forceinline__ void horizontal_moments_in_place(float *lds, const Taps &taps) {
    constexpr int IH = TH + 10, IP = in_pitch<TW>(), QW = TW / 4, PL = IH * TW;
    constexpr int ITEMS = IH * QW;
    static_assert(ITEMS <= 2 * NT, "at most two horizontal items per thread");
    const float *sx = lds, *sy = lds + IH * IP;
    const int i1 = threadIdx.x, i2 = threadIdx.x + NT;
    const bool has1 = i1 < ITEMS, has2 = i2 < ITEMS;
    const int r1 = i1 / QW, c1 = (i1 - r1 * QW) * 4;
    const int r2 = i2 / QW, c2 = (i2 - r2 * QW) * 4;
    float m[NP][4];
    float a[14], b[14];
    if (has1) {
        h_item_load(sx + r1 * IP + c1, sy + r1 * IP + c1, a, b);
        h_item_compute<NP>(a, b, taps, m);
    }
    if (has2) h_item_load(sx + r2 * IP + c2, sy + r2 * IP + c2, a, b);
    __syncthreads();  // every read of the staged tile is done
    if (has1) {
        const int o = r1 * TW + c1;
#pragma unroll
        for (int p = 0; p < NP; ++p)
            *reinterpret_cast<float4 *>(lds + p * PL + o) = make_float4(m[p][0], m[p][1], m[p][2], m[p][3]);
    }
    if (has2) {
        h_item_compute<NP>(a, b, taps, m);
        const int o = r2 * TW + c2;
#pragma unroll
        for (int p = 0; p < NP; ++p)
            *reinterpret_cast<float4 *>(lds + p * PL + o) = make_float4(m[p][0], m[p][1], m[p][2], m[p][3]);
    }
    __syncthreads();
}

// Vertical pass: for RB stacked map rows of one tile column at a time, the
// NP moments from RB + 10 values of each horizontal plane (FMA order
// k = 0..10), handed to `fn(r, c, m)` (m: the NP moments of the pixel) for
// every map pixel inside the valid region (x0 + c < MW, y0 + r < MH).
template <int TW, int TH, int NT, int RB, int NP, typename F>
__device__ __forceinline__ void vertical_moments(const float *hm, const Taps &taps, int x0, int y0, int MW,
                                                 int MH, F &&fn) {
    static_assert(TH % RB == 0, "tile height must be a multiple of the row block");
    constexpr int IH = TH + 10, PL = IH * TW;
    for (int it = threadIdx.x; it < (TH / RB) * TW; it += NT) {
        const int c = it % TW, r0 = (it / TW) * RB;
        if (x0 + c >= MW || y0 + r0 >= MH) continue;
        float m[RB][NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            float v[RB + 10];
#pragma unroll
            for (int i = 0; i < RB + 10; ++i) v[i] = hm[p * PL + (r0 + i) * TW + c];
#pragma unroll
            for (int j = 0; j < RB; ++j) {
                float acc = 0.f;
#pragma unroll
                for (int k = 0; k < 11; ++k) acc = fmaf(taps.g[k], v[j + k], acc);
                m[j][p] = acc;
            }
        }
#pragma unroll
        for (int j = 0; j < RB; ++j)
            if (y0 + r0 + j < MH) fn(r0 + j, c, m[j]);
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

// v plus lane (lane ^ 1), (lane ^ 2), or the lane mirrored in its row of 8
// or 16 lanes, as one DPP add.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_add(float v) {
    const int o = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, kRowMask, 0xF, false);
    return v + __builtin_bit_cast(float, o);
}

// Sum over the 64 lanes of a wave in fp32, in a fixed order: pairs, quads
// (DPP quad permutations), rows of 8 and 16 (row half-mirror and mirror), then
// row 0 into row 1 and row 2 into row 3 (row broadcast 15), then rows 0-1 into
// rows 2-3 (row broadcast 31).  The total is in lane 63 and returned to every
// lane (a wave-uniform value).
__device__ __forceinline__ float wave_sum_f32(float v) {
    v = dpp_add<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
    v = dpp_add<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
    v = dpp_add<0x141, 0xF>(v);  // row_half_mirror
    v = dpp_add<0x140, 0xF>(v);  // row_mirror
    v = dpp_add<0x142, 0xA>(v);  // row_bcast15 into rows 1 and 3
    v = dpp_add<0x143, 0xC>(v);  // row_bcast31 into rows 2 and 3
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
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
