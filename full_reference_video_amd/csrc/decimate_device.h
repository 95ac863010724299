// decimate_device.h — exact box low-pass and decimate for gfx950 (device
// code, library-private; the decimation role of the float_ssim step kernel).
//
// "ADR-1405: float_ssim_hip decimates on the device, bit-identical to the
// CPU", Context and Decision 1: output (X, Y) of a plane is the window at
// (X*s + i, Y*s + j), i, j in [-s/2, s-1-s/2], half-sample symmetric edges,
// of the fp32 products v * tap (tap = 1.0f/(s*s) formed on the host), summed
// exactly and rounded once to fp32.  The pages keep the exact sum as an int64
// count of 2^-52 units (every product is a multiple of 2^-45 and the sum stays
// below 2^8, so it fits for s <= 128).  Here it is kept wherever it is
// cheapest, always exactly:
//
// Three code paths compute that same exact sum:
//
//  * general_block — any s <= 128: each product is formed in fp32 and the
//    products are summed exactly in fp64 (the bound is at the function).
//
//  * pow2_scalar_block — s = 2^k on planes whose rows are not 16-byte
//    aligned: the plain integer sum of the raw samples, read one by one.
//
//  * pow2_wave — s = 2^k, where tap = 2^-2k and every product is exact,
//    so a product is raw * 2^-(2k + bpc - 8): a constant scaling of the raw
//    integer.  The scaling is hoisted out of the window sum,
//    which becomes a plain integer sum of raw samples (v_sad_u8 / v_sad_u16
//    add four or two samples per instruction), rounded once to fp32 and
//    scaled by the exact power of two.  This is the HBM-bound path of the
//    1080p and 2160p frames.
//
// Layout of pow2_wave.  Chunk k of a row is the s raw columns
// [k*s, k*s + s); window X covers the high half of chunk X-1 and the low half
// of chunk X.  A lane owns one aligned group of G = max(s, 16/sizeof(T))
// columns (CPT = G/s chunks) and reads it with 128-bit non-temporal loads for
// each of the s rows of the window band, so a wave reads contiguous,
// 16-byte-aligned kilobytes.  The high half of the chunk before a lane's
// first chunk comes from the previous lane (one cross-lane shift).  To make
// every wave self-contained, wave v's lanes hold groups 63v-1 .. 63v+62: lane
// 0 re-reads the last group of the previous wave (1/64 extra, which the XCD
// remap keeps in the same L2) and outputs nothing.  At the left edge lane 0
// of wave 0 stands in for group -1 with the mirror of chunk 0's low half.
#pragma once

#include "vqm_kernels.h"

namespace vqm {
namespace dec {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Half-sample symmetric extension (-1 -> 0, n -> n-1), repeated as often as
// needed: the periodic even extension with period 2n.  No loop.
__device__ __forceinline__ int mirror(int i, int n) {
    if (i >= 0 && i < n) return i;
    const int p = 2 * n;
    int m = i % p;
    if (m < 0) m += p;
    return m < n ? m : p - 1 - m;
}

// ------------------------------------------------------------ general path

// One 256-thread block of the general kernel: outputs (64 bx + lane,
// 4 by + wave).
template <typename T>
__device__ __forceinline__ void general_block(const DecimateFrame &fr, int bx, int by, int w, int h, int bpc,
                                              int s, float tap, int dec_w, int dec_h, int opitch, bool packed) {
    const T *__restrict__ ref = static_cast<const T *>(fr.ref);
    const T *__restrict__ dis = static_cast<const T *>(fr.dis);
    const int X = bx * 64 + (threadIdx.x & 63);
    const int Y = by * 4 + (threadIdx.x >> 6);
    if (X >= dec_w || Y >= dec_h) return;
    const int x0 = X * s - s / 2, y0 = Y * s - s / 2;
    // The exact sum of the fp32 products raw * tap, accumulated in fp64: every
    // product is a multiple of ulp(tap) = 2^(e - 23) (tap in [2^e, 2^(e+1)),
    // e = -ceil(2 log2 s)) and the window's sum stays below 2^bpc, so every
    // partial sum is an integer multiple of ulp(tap) below
    // 2^(bpc + 23 + ceil(2 log2 s)) <= 2^53 for bpc <= 16 and s <= 128: fp64
    // holds it exactly, as the int64 count of 2^-52 units does.
    // Every partial sum of any subset of the products is exact too, so the
    // order of the additions is free: four independent sums per plane keep
    // four loads in flight.
    double ar = 0.0, ad = 0.0;
    if (x0 >= 0 && x0 + s <= w && y0 >= 0 && y0 + s <= h) {
        const T *pr = ref + (size_t)y0 * (size_t)w + x0;
        const T *pd = dis + (size_t)y0 * (size_t)w + x0;
        double a4[4] = {0.0, 0.0, 0.0, 0.0}, d4[4] = {0.0, 0.0, 0.0, 0.0};
        for (int j = 0; j < s; ++j, pr += w, pd += w) {
            int i = 0;
            for (; i + 4 <= s; i += 4) {
                T rv[4], dv[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    rv[k] = pr[i + k];
                    dv[k] = pd[i + k];
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    a4[k] += (double)((float)rv[k] * tap);
                    d4[k] += (double)((float)dv[k] * tap);
                }
            }
            for (; i < s; ++i) {
                a4[0] += (double)((float)pr[i] * tap);
                d4[0] += (double)((float)pd[i] * tap);
            }
        }
        ar = (a4[0] + a4[1]) + (a4[2] + a4[3]);
        ad = (d4[0] + d4[1]) + (d4[2] + d4[3]);
    } else {
        for (int j = 0; j < s; ++j) {
            const size_t row = (size_t)mirror(y0 + j, h) * (size_t)w;
            for (int i = 0; i < s; ++i) {
                const int xx = mirror(x0 + i, w);
                ar += (double)((float)ref[row + xx] * tap);
                ad += (double)((float)dis[row + xx] * tap);
            }
        }
    }
    const size_t o = (size_t)Y * opitch + X;
    if (packed) {
        // s = 2^k: tap = 2^-2k and the sum times s^2 is the raw integer sum.
        const double ss = (double)s * (double)s;
        static_cast<uint16_t *>(fr.out_ref)[o] = (uint16_t)(ar * ss);
        static_cast<uint16_t *>(fr.out_dis)[o] = (uint16_t)(ad * ss);
        return;
    }
    // One rounding to fp32, then the exact scaling of the samples to 8 bits.
    static_cast<float *>(fr.out_ref)[o] = ldexpf((float)ar, 8 - bpc);
    static_cast<float *>(fr.out_dis)[o] = ldexpf((float)ad, 8 - bpc);
}

// One 256-thread block of the power-of-two path for planes whose rows are not
// 16-byte aligned (odd widths): outputs (64 bx + lane, 4 by + wave), each
// the integer sum of its S x S raw samples, read one by one (every product
// v * tap is exact at s = 2^k, so the window sum is sum(raw) * post).  The
// mirrored row and column of each window position are found once.
template <typename T, int S>
__device__ __forceinline__ void pow2_scalar_block(const DecimateFrame &fr, int bx, int by, int w, int h,
                                                  int dec_w, int dec_h, int opitch, float post, bool packed) {
    const T *__restrict__ ref = static_cast<const T *>(fr.ref);
    const T *__restrict__ dis = static_cast<const T *>(fr.dis);
    const int X = bx * 64 + (threadIdx.x & 63);
    const int Y = by * 4 + (threadIdx.x >> 6);
    if (X >= dec_w || Y >= dec_h) return;
    int col[S];
    size_t row[S];
#pragma unroll
    for (int i = 0; i < S; ++i) {
        col[i] = mirror(X * S - S / 2 + i, w);
        row[i] = (size_t)mirror(Y * S - S / 2 + i, h) * (size_t)w;
    }
    uint32_t ar = 0, ad = 0;
#pragma unroll
    for (int j = 0; j < S; ++j)
#pragma unroll
        for (int i = 0; i < S; ++i) {
            ar += ref[row[j] + col[i]];
            ad += dis[row[j] + col[i]];
        }
    const size_t o = (size_t)Y * opitch + X;
    if (packed) {
        static_cast<uint16_t *>(fr.out_ref)[o] = (uint16_t)ar;
        static_cast<uint16_t *>(fr.out_dis)[o] = (uint16_t)ad;
    } else {
        // One rounding of the exact sum (uint32 -> fp32 is RNE), then the
        // exact power of two.
        static_cast<float *>(fr.out_ref)[o] = (float)ar * post;
        static_cast<float *>(fr.out_dis)[o] = (float)ad * post;
    }
}

// ------------------------------------------------------------ power-of-two path

template <typename T> struct Samples;
template <> struct Samples<uint8_t> {
    static constexpr int per_word = 4;
    // sum of the four bytes of w, plus acc
    __device__ static uint32_t add(uint32_t w, uint32_t acc) { return __builtin_amdgcn_sad_u8(w, 0u, acc); }
};
template <> struct Samples<uint16_t> {
    static constexpr int per_word = 2;
    // sum of the two halves of w, plus acc
    __device__ static uint32_t add(uint32_t w, uint32_t acc) { return __builtin_amdgcn_sad_u16(w, 0u, acc); }
};

// Bit mask selecting samples [e0, e1) of a 32-bit word of T samples.
template <typename T>
__host__ __device__ constexpr uint32_t sample_mask(int e0, int e1) {
    uint32_t m = 0;
    for (int e = e0; e < e1; ++e) m |= (uint32_t)((1ull << (8 * sizeof(T))) - 1) << (8 * sizeof(T) * e);
    return m;
}

// Add the samples of a word whose first sample is column g0 of the lane's
// group into the half sums of the chunks they belong to.  Everything but
// `word` is a compile-time constant after unrolling.
template <typename T, int S, int CPT>
__device__ __forceinline__ void add_word(uint32_t word, int g0, uint32_t (&lo)[CPT], uint32_t (&hi)[CPT]) {
    constexpr int SPW = Samples<T>::per_word;
    constexpr int HALF = S / 2;
    if constexpr (HALF >= SPW) {
        const int k = g0 / S;
        if ((g0 % S) >= HALF) hi[k] = Samples<T>::add(word, hi[k]);
        else lo[k] = Samples<T>::add(word, lo[k]);
    } else {
        // A word spans several half-chunks: split it by masks.
#pragma unroll
        for (int e0 = 0; e0 < SPW; e0 += HALF) {
            const int g = g0 + e0;
            const int k = g / S;
            const uint32_t part = word & sample_mask<T>(e0, e0 + HALF);
            if ((g % S) >= HALF) hi[k] = Samples<T>::add(part, hi[k]);
            else lo[k] = Samples<T>::add(part, lo[k]);
        }
    }
}

template <typename T, int S> struct Pow2Shape {
    static constexpr int SPW = Samples<T>::per_word;  // samples per 32-bit word
    static constexpr int V = 4 * SPW;                 // samples per 128-bit load
    static constexpr int G = S > V ? S : V;           // raw columns per lane
    static constexpr int NV = G / V;                  // 128-bit loads per lane per row
    static constexpr int CPT = G / S;                 // chunks (outputs) per lane
};

// One wave of the power-of-two kernel: wave wv of output row Y.
template <typename T, int S>
__device__ __forceinline__ void pow2_wave(const DecimateFrame &fr, int wv, int Y, int w, int h, int dec_w,
                                          float post, int opitch, bool packed) {
    using Sh = Pow2Shape<T, S>;
    constexpr int V = Sh::V, NV = Sh::NV, CPT = Sh::CPT, G = Sh::G;
    constexpr int HALF = S / 2;
    const T *__restrict__ ref = static_cast<const T *>(fr.ref);
    const T *__restrict__ dis = static_cast<const T *>(fr.dis);

    const int lane = threadIdx.x & 63;
    const int g = 63 * wv + lane - 1;  // this lane's group; -1 stands for the left mirror
    const int c0 = (g < 0 ? 0 : g) * G;

    uint32_t lr[CPT], hr[CPT], ld[CPT], hd[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) lr[k] = hr[k] = ld[k] = hd[k] = 0u;

    constexpr int kRowUnroll = S <= 16 ? S : 4;
#pragma unroll kRowUnroll
    for (int r = 0; r < S; ++r) {
        const size_t row = (size_t)mirror(Y * S - HALF + r, h) * (size_t)w;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            // w is a multiple of V, so a vector is wholly inside or outside
            // the row.  A vector outside reads the row's last vector instead
            // (no branch: a load under a per-lane branch makes the compiler
            // wait for every earlier load first).  Its samples land only in
            // the high half of the last chunk or in chunks past it, that is
            // in outputs X >= dec_w, which are never stored: the fast path
            // keeps the last window's low half inside the row.
            const int col = c0 + v * V < w ? c0 + v * V : w - V;
            const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(ref + row + col));
            const u32x4 d = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(dis + row + col));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                add_word<T, S, CPT>(a[q], v * V + q * Sh::SPW, lr, hr);
                add_word<T, S, CPT>(d[q], v * V + q * Sh::SPW, ld, hd);
            }
        }
    }
    if (g < 0) {
        // Columns -s/2..-1 mirror onto 0..s/2-1: the low half of chunk 0.
        hr[CPT - 1] = lr[0];
        hd[CPT - 1] = ld[0];
    }
    // High half of the chunk just before this lane's first chunk.
    const uint32_t pr = __shfl_up(hr[CPT - 1], 1, 64);
    const uint32_t pd = __shfl_up(hd[CPT - 1], 1, 64);
    if (lane == 0) return;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const int X = g * CPT + k;
        if (X < dec_w) {
            const uint32_t tr = (k == 0 ? pr : hr[k - 1]) + lr[k];
            const uint32_t td = (k == 0 ? pd : hd[k - 1]) + ld[k];
            const size_t o = (size_t)Y * opitch + X;
            if (packed) {
                // The raw sums themselves (below 2^16 when packed).
                static_cast<uint16_t *>(fr.out_ref)[o] = (uint16_t)tr;
                static_cast<uint16_t *>(fr.out_dis)[o] = (uint16_t)td;
            } else {
                // One rounding (the only one: sums below 2^24 are exact),
                // then the exact power of two.
                static_cast<float *>(fr.out_ref)[o] = (float)tr * post;
                static_cast<float *>(fr.out_dis)[o] = (float)td * post;
            }
        }
    }
}

}  // namespace dec
}  // namespace vqm
