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
//  * general_rows_block — any s <= 128: each product's exact integer count
//    of units, formed with one fused multiply-add, summed as integers over
//    the window into the int64 count of 2^-52 units (the bound is at the
//    function); lanes read consecutive columns.  No fp64 anywhere, as the
//    ADR's contract for the decimation asks.
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

// Raw columns one workgroup of the general path covers per output row (four
// per thread of 256), and the windows that makes: K windows of s columns,
// K s <= kGenCols, at most one window per thread.
constexpr int kGenThreads = 256;
constexpr int kGenJ = 4;
constexpr int kGenCols = kGenJ * kGenThreads;
__host__ __device__ inline int gen_windows_per_block(int s) {
    const int k = kGenCols / s;
    return k < 1 ? 1 : (k > kGenThreads ? kGenThreads : k);
}
// LDS ints the general path needs: per plane a column's raw sum and its
// error sum.
constexpr int kGenLdsInts = 4 * kGenCols;

// The s rows of a window band, summed per column.  sr: the raw samples (exact
// integers); er: the errors raw * m - fl(raw * m) of the products by the
// tap's significand m (exact integers, |sum| <= 2^22, so exact in fp32).
template <typename T>
struct GenColumns {
    uint32_t sr[kGenJ], sd[kGenJ];
    float er[kGenJ], ed[kGenJ];
    // Rows are loaded in groups of U before any of them is added, so the
    // group's 8 U loads are in flight together (the compiler keeps loads and
    // arithmetic in source order row by row otherwise).
    template <int U>
    __device__ __forceinline__ void add_rows(const T *__restrict__ rrow, const T *__restrict__ drow, size_t w,
                                             const int (&col)[kGenJ], float m) {
        uint32_t a[U][kGenJ], d[U][kGenJ];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < kGenJ; ++j) {
                a[u][j] = rrow[u * w + col[j]];
                d[u][j] = drow[u * w + col[j]];
            }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < kGenJ; ++j) {
                const float fa = (float)a[u][j], fd = (float)d[u][j];
                const float qa = fa * m, qd = fd * m;
                er[j] += fmaf(fa, m, -qa);
                ed[j] += fmaf(fd, m, -qd);
                sr[j] += a[u][j];
                sd[j] += d[u][j];
            }
    }
};

// One workgroup of the general path: windows X0 .. X0 + K - 1 of output row Y
// (X0 = seg K), any s <= 128.
//
// The exact window sum without fp64: with tap = M 2^(e - 23) (M its 24-bit
// significand) every product is fl(raw * 2^-(bpc-8) * tap) = q 2^E with
// q = fl(raw * M) and E = e - 23 - (bpc - 8) (scaling by a power of two
// commutes with the rounding).  raw * M is an integer below 2^40, so q is one
// too and its error r = raw * M - q, formed exactly by one fused multiply-add,
// is an integer with |r| <= 2^15.  The window's sum of q is therefore the
// integer M * sum(raw) - sum(r), exact in int64 (below 2^54); shifted into
// units of 2^-52 (the shift E + 52 is >= 7) it is the pages' int64 window
// sum, converted once to fp32.  Per column the s errors add exactly in fp32
// (|sum| <= 2^22, integers), then as int32 over the window (|sum| <= 2^29).
//
// Layout: thread t owns the virtual columns cs + t + 256 j (j < 4) of the
// band (cs = X0 s - s/2), each read from its mirrored raw column, so a wave's
// loads of one raw row are consecutive samples.  It sums its columns over the
// s rows of the band (the same rows for the whole workgroup: a scalar row
// pointer, four rows of loads in flight), the column sums meet in LDS, and
// thread k forms window X0 + k from its s consecutive virtual columns.
template <typename T>
__device__ __forceinline__ void general_rows_block(const DecimateFrame &fr, int seg, int Y, int w, int h, int bpc,
                                                   int s, float tap, int dec_w, int opitch, bool packed,
                                                   int *lds) {
    const T *__restrict__ ref = static_cast<const T *>(fr.ref);
    const T *__restrict__ dis = static_cast<const T *>(fr.dis);
    const int K = gen_windows_per_block(s);
    const int X0 = seg * K;
    const int ncols = K * s;
    const int cs = X0 * s - s / 2;
    const int t = threadIdx.x;
    const uint32_t tb = __float_as_uint(tap);
    const uint32_t m_int = (tb & 0x7fffffu) | 0x800000u;
    const float m = (float)m_int;  // exact: below 2^24
    const int shift = (int)((tb >> 23) & 0xffu) - 127 - 23 - (bpc - 8) + 52;

    // Every load is unconditional: a column the thread does not own reads a
    // mirrored column in the plane, and its sums are never stored.
    int col[kGenJ];
#pragma unroll
    for (int j = 0; j < kGenJ; ++j) col[j] = mirror(cs + t + kGenThreads * j, w);
    GenColumns<T> acc;
#pragma unroll
    for (int j = 0; j < kGenJ; ++j) {
        acc.sr[j] = acc.sd[j] = 0u;
        acc.er[j] = acc.ed[j] = 0.f;
    }
    const int y0 = Y * s - s / 2;
    if (y0 >= 0 && y0 + s <= h) {
        // Inside the plane: rows y0 .. y0 + s - 1, no mirror.
        const T *rrow = ref + (size_t)y0 * (size_t)w, *drow = dis + (size_t)y0 * (size_t)w;
        int r = 0;
        for (; r + 4 <= s; r += 4, rrow += 4 * (size_t)w, drow += 4 * (size_t)w)
            acc.template add_rows<4>(rrow, drow, (size_t)w, col, m);
        // the last s % 4 rows as one group as well
        switch (s - r) {
        case 3: acc.template add_rows<3>(rrow, drow, (size_t)w, col, m); break;
        case 2: acc.template add_rows<2>(rrow, drow, (size_t)w, col, m); break;
        case 1: acc.template add_rows<1>(rrow, drow, (size_t)w, col, m); break;
        default: break;
        }
    } else {
        for (int r = 0; r < s; ++r) {
            const size_t row = (size_t)mirror(y0 + r, h) * (size_t)w;
            acc.template add_rows<1>(ref + row, dis + row, (size_t)w, col, m);
        }
    }
    int *col_sr = lds, *col_sd = lds + kGenCols, *col_er = lds + 2 * kGenCols, *col_ed = lds + 3 * kGenCols;
#pragma unroll
    for (int j = 0; j < kGenJ; ++j) {
        const int v = t + kGenThreads * j;
        if (v < ncols) {
            col_sr[v] = (int)acc.sr[j];
            col_sd[v] = (int)acc.sd[j];
            col_er[v] = (int)acc.er[j];
            col_ed[v] = (int)acc.ed[j];
        }
    }
    __syncthreads();
    const int X = X0 + t;
    if (t < K && X < dec_w) {
        int sumr = 0, sumd = 0, errr = 0, errd = 0;
        for (int i = 0; i < s; ++i) {
            sumr += col_sr[t * s + i];
            sumd += col_sd[t * s + i];
            errr += col_er[t * s + i];
            errd += col_ed[t * s + i];
        }
        const size_t o = (size_t)Y * opitch + X;
        if (packed) {
            // s = 2^k: every product is exact and the sum is sum(raw) 2^-2k.
            static_cast<uint16_t *>(fr.out_ref)[o] = (uint16_t)sumr;
            static_cast<uint16_t *>(fr.out_dis)[o] = (uint16_t)sumd;
        } else {
            const long long qr = (long long)m_int * (long long)(uint32_t)sumr - (long long)errr;
            const long long qd = (long long)m_int * (long long)(uint32_t)sumd - (long long)errd;
            // the int64 count of 2^-52 units, one rounding to fp32, then the
            // exact power of two
            static_cast<float *>(fr.out_ref)[o] = ldexpf((float)(qr << shift), -52);
            static_cast<float *>(fr.out_dis)[o] = ldexpf((float)(qd << shift), -52);
        }
    }
    __syncthreads();  // the LDS is reused by the workgroup's next role or unit
}

// Output rows each thread of the scalar power-of-two path sums (of one output
// column): enough that a thread has 32 or more raw samples of both planes in
// flight at s = 2 and 4 (a workgroup with one 2 x 2 window per thread reads
// too little to hide the memory latency).
template <int S>
__host__ __device__ constexpr int scalar_rows_per_thread() {
    return S == 2 ? 4 : (S == 4 ? 2 : 1);
}

// One 256-thread block of the power-of-two path for planes whose rows are not
// 16-byte aligned (odd widths): output column 64 bx + lane, output rows
// RPT (4 by + wave) .. + RPT - 1, each the integer sum of its S x S raw
// samples, read one by one (every product v * tap is exact at s = 2^k, so
// the window sum is sum(raw) * post).  The mirrored rows and columns are
// found once, and every sample of the thread's windows is loaded before any
// is added.
template <typename T, int S>
__device__ __forceinline__ void pow2_scalar_block(const DecimateFrame &fr, int bx, int by, int w, int h,
                                                  int dec_w, int dec_h, int opitch, float post, bool packed) {
    constexpr int RPT = scalar_rows_per_thread<S>();
    const T *__restrict__ ref = static_cast<const T *>(fr.ref);
    const T *__restrict__ dis = static_cast<const T *>(fr.dis);
    const int X = bx * 64 + (threadIdx.x & 63);
    const int Y0 = (by * 4 + (threadIdx.x >> 6)) * RPT;
    if (X >= dec_w || Y0 >= dec_h) return;
    int col[S];
    size_t row[RPT * S];  // the window rows of outputs Y0 .. Y0 + RPT - 1, in order
#pragma unroll
    for (int i = 0; i < S; ++i) col[i] = mirror(X * S - S / 2 + i, w);
#pragma unroll
    for (int q = 0; q < RPT * S; ++q) row[q] = (size_t)mirror(Y0 * S - S / 2 + q, h) * (size_t)w;
    uint32_t ar[RPT], ad[RPT];
    if constexpr (RPT * S * S <= 16) {
        // All of them in flight at once (a row past the plane reads a mirrored
        // row inside it; its output is not stored).
        T va[RPT * S][S], vd[RPT * S][S];
#pragma unroll
        for (int q = 0; q < RPT * S; ++q)
#pragma unroll
            for (int i = 0; i < S; ++i) {
                va[q][i] = ref[row[q] + col[i]];
                vd[q][i] = dis[row[q] + col[i]];
            }
#pragma unroll
        for (int k = 0; k < RPT; ++k) {
            ar[k] = ad[k] = 0u;
#pragma unroll
            for (int j = 0; j < S; ++j)
#pragma unroll
                for (int i = 0; i < S; ++i) {
                    ar[k] += va[k * S + j][i];
                    ad[k] += vd[k * S + j][i];
                }
        }
    } else {
#pragma unroll
        for (int k = 0; k < RPT; ++k) {
            ar[k] = ad[k] = 0u;
#pragma unroll
            for (int j = 0; j < S; ++j)
#pragma unroll
                for (int i = 0; i < S; ++i) {
                    ar[k] += ref[row[k * S + j] + col[i]];
                    ad[k] += dis[row[k * S + j] + col[i]];
                }
        }
    }
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
        if (Y0 + k >= dec_h) break;
        const size_t o = (size_t)(Y0 + k) * opitch + X;
        if (packed) {
            static_cast<uint16_t *>(fr.out_ref)[o] = (uint16_t)ar[k];
            static_cast<uint16_t *>(fr.out_dis)[o] = (uint16_t)ad[k];
        } else {
            // One rounding of the exact sum (uint32 -> fp32 is RNE), then the
            // exact power of two.
            static_cast<float *>(fr.out_ref)[o] = (float)ar[k] * post;
            static_cast<float *>(fr.out_dis)[o] = (float)ad[k] * post;
        }
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

// N 32-bit words to a 4N-byte aligned address in 16-byte (or smaller) stores.
template <int N>
__device__ __forceinline__ void store_words(void *p, const uint32_t (&w)[N]) {
    if constexpr (N == 1) {
        *static_cast<uint32_t *>(p) = w[0];
    } else if constexpr (N == 2) {
        *static_cast<uint2 *>(p) = make_uint2(w[0], w[1]);
    } else {
        static_assert(N % 4 == 0, "whole 16-byte groups");
#pragma unroll
        for (int i = 0; i < N / 4; ++i)
            static_cast<uint4 *>(p)[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
    }
}

// The windows of one unit from its half-chunk sums: the high half before a
// lane's first chunk comes from the previous lane (one cross-lane shift);
// store them.
template <typename T, int S>
__device__ __forceinline__ void pow2_finish(const DecimateFrame &fr, int wv, int Y, int dec_w, float post,
                                            int opitch, bool packed, uint32_t (&lr)[Pow2Shape<T, S>::CPT],
                                            uint32_t (&hr)[Pow2Shape<T, S>::CPT], uint32_t (&ld)[Pow2Shape<T, S>::CPT],
                                            uint32_t (&hd)[Pow2Shape<T, S>::CPT]) {
    constexpr int CPT = Pow2Shape<T, S>::CPT;
    const int lane = threadIdx.x & 63;
    const int g = 63 * wv + lane - 1;
    if (g < 0) {
        // Columns -s/2..-1 mirror onto 0..s/2-1: the low half of chunk 0.
        hr[CPT - 1] = lr[0];
        hd[CPT - 1] = ld[0];
    }
    // High half of the chunk just before this lane's first chunk.
    const uint32_t pr = __shfl_up(hr[CPT - 1], 1, 64);
    const uint32_t pd = __shfl_up(hd[CPT - 1], 1, 64);
    if (lane == 0) return;
    if constexpr (CPT >= 2) {
        // A lane's CPT adjacent outputs in one store per plane where they are
        // all inside the row (the planes are 16-byte aligned and their pitch
        // a multiple of 8 outputs), so a unit issues two stores instead of
        // 2 CPT.
        const int X0 = g * CPT;
        if (X0 + CPT <= dec_w) {
            uint32_t tr[CPT], td[CPT];
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                tr[k] = (k == 0 ? pr : hr[k - 1]) + lr[k];
                td[k] = (k == 0 ? pd : hd[k - 1]) + ld[k];
            }
            const size_t o = (size_t)Y * opitch + X0;
            if (packed) {
                uint32_t wr[CPT / 2], wd[CPT / 2];
#pragma unroll
                for (int k = 0; k < CPT / 2; ++k) {
                    wr[k] = tr[2 * k] | (tr[2 * k + 1] << 16);
                    wd[k] = td[2 * k] | (td[2 * k + 1] << 16);
                }
                store_words<CPT / 2>(static_cast<uint16_t *>(fr.out_ref) + o, wr);
                store_words<CPT / 2>(static_cast<uint16_t *>(fr.out_dis) + o, wd);
            } else {
                uint32_t wr[CPT], wd[CPT];
#pragma unroll
                for (int k = 0; k < CPT; ++k) {
                    wr[k] = __builtin_bit_cast(uint32_t, (float)tr[k] * post);
                    wd[k] = __builtin_bit_cast(uint32_t, (float)td[k] * post);
                }
                store_words<CPT>(static_cast<float *>(fr.out_ref) + o, wr);
                store_words<CPT>(static_cast<float *>(fr.out_dis) + o, wd);
            }
            return;
        }
    }
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

// One wave of the power-of-two kernel: wave wv of output row Y (rows
// streamed: each row's loads are added as they arrive, so any S fits).
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
    pow2_finish<T, S>(fr, wv, Y, dec_w, post, opitch, packed, lr, hr, ld, hd);
}

}  // namespace dec
}  // namespace vqm
