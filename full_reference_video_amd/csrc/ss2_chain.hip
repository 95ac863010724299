// ss2_chain.hip — the ssimulacra2 per-scale chain on the device: the three
// multiplies, the recursive blur along every row and then every column, the
// statistics of the blurred planes, and the 2x2 downsample between scales.
//
// "Research-1363: Device-resident ssimulacra2 and a single-wait MS-SSIM on
// SYCL", Finding 2: with contraction off and every product its own rounded
// value, the multiplies, both blur passes and the downsample reproduce the
// CPU bit for bit; Finding 7: the blur is a sequential recurrence along each
// line, so a pass has one work-item per row or column, five blurs per
// channel and scale; Finding 4: the six sums per channel come from exact
// fp32 pairs in a fixed tree.  The recursion (third order, caller
// coefficients B, a1, a2, a3, at rest outside the line), causal then
// anticausal:
//   w[i] = ((B x[i] + a3 w[i-3]) + a2 w[i-2]) + a1 w[i-1]
//   y[i] = ((B w[i] + a3 y[i+3]) + a2 y[i+2]) + a1 y[i+1]
// (the library is compiled with -ffp-contract=off, so each product here is
// rounded on its own).
//
// The work is a set of independent sequential walks, one per line, plane,
// channel and scale, so it is laid out for them:
//  * Every scale runs in one launch per pass.  The downsampled images come
//    first (the pyramid of the two pictures needs no blur), so the short
//    lines of the small scales run beside the long ones of the first scale
//    instead of after them.
//  * A workgroup is four waves, one per SIMD.  The row pass holds 51 rows of
//    all five planes in its 256 lanes (255 used), so no SIMD carries two
//    walkers while the others wait at a barrier.  The column pass holds 32
//    columns of all five planes (160 lanes walk, all 256 form the
//    statistics): its loads are then whole 128-byte lines, where 51-column
//    blocks shared lines with their neighbours and fetched 1.6 times the
//    bytes they used.
//  * No pass writes the causal outputs w: the causal walk keeps only its
//    state (w[i-1], w[i-2], w[i-3]) at the end of every 32-sample chunk, and
//    the anticausal walk, chunk by chunk from the end, recomputes the
//    chunk's w from that state (the same operations on the same values, so
//    the same bits) and walks back over it in registers.
//  * Row pass: chunks of the two images are loaded two ahead into
//    registers, staged through LDS row-contiguously (the page's horizontal
//    walk made every lane of a load touch its own cache line), and each
//    lane reads its row's samples there, times its plane's second factor
//    (the other image for the products, a row of ones for a and b), so the
//    multiplies cost no pass.  Outputs go back through LDS.
//  * Column pass: lanes own columns (loads contiguous across a lane group);
//    each 32-row chunk's five blurred planes meet in LDS and the chunk's
//    pixels go straight into the statistics, so the blurred planes are never
//    written.  One more small launch sums each (scale, channel)'s partials.
#include "ss2_pairs.h"
#include "ss2_kernels.h"

#include <algorithm>
#include <type_traits>

namespace vqm {
namespace {

using namespace ss2;

constexpr int kChunk = 32;          // samples of a line per chunk
constexpr int kPitch = kChunk + 1;  // odd pitch: lanes reading along their own rows hit distinct banks
constexpr int kRing = 3;            // register sets: one chunk in use, two loading

struct Coef {
    float B, a1, a2, a3;
};

template <int V>
using Ic = std::integral_constant<int, V>;

// Lines per workgroup and threads: five planes of 51 lines in four waves,
// or one plane of 64 lines in one wave.
template <int NP>
struct Shape {
    static constexpr int kRowLines = NP == 5 ? 51 : 64;  // rows per row-pass workgroup (5 x 51 of 256 lanes)
    static constexpr int kColLines = NP == 5 ? 32 : 64;  // columns per column-pass workgroup (128-byte rows)
    static constexpr int kThreads = NP == 5 ? 256 : 64;
    static constexpr int kState = 3 * kThreads;  // floats of one checkpoint
    static constexpr int kRowChunk = NP == 5 ? 64 : 32;  // columns per chunk of the row pass
};

// One step of the recursion: s1, s2, s3 are the newest, second and third
// newest states; the sum adds the oldest first.
__device__ __forceinline__ float recur(const Coef &k, float x, float s1, float s2, float s3) {
    const float in = k.B * x;
    const float t3 = k.a3 * s3;
    const float t2 = k.a2 * s2;
    const float t1 = k.a1 * s1;
    return ((in + t3) + t2) + t1;
}

struct State {
    float s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
    __device__ __forceinline__ float step(const Coef &k, float x) {
        const float y = recur(k, x, s1, s2, s3);
        s3 = s2;
        s2 = s1;
        s1 = y;
        return y;
    }
};

// N steps over values held in registers, replaced by the outputs; forward
// (index 0 first) or backward (index N - 1 first).
template <int N, bool Back>
__device__ __forceinline__ void walk_regs(const Coef &k, float (&v)[N], State &st) {
#pragma unroll
    for (int jj = 0; jj < N; ++jj) {
        const int j = Back ? N - 1 - jj : jj;
        v[j] = st.step(k, v[j]);
    }
}

// One scale of the chain: its size, its images, its row-blurred planes
// (NP per channel, pstride apart), and where its workgroups, checkpoints and
// partials start.
struct ScaleDesc {
    int w, h;
    long long pstride;
    const float *a[kSs2MaxChannels], *b[kSs2MaxChannels];
    float *rows[kSs2MaxChannels];
    float *out[kSs2MaxChannels];       // column pass output (NULL: statistics only)
    int row_block0, col_block0;        // first workgroup of the scale in each pass
    long long ckpt_rows0, ckpt_cols0;  // first checkpoint float of the scale
    int part0;                         // first partial of the scale
};

struct Chain {
    ScaleDesc s[kSs2MaxScales];
    int nscales, nch;
    float *ckpt;
    Pair *partials;  // NULL: no statistics
    double *result;  // 6 doubles per (scale, channel)
};

// The scale of a workgroup (scales in order, first scale's blocks first).
__device__ __forceinline__ int scale_of(const Chain &ch, int block, bool cols) {
    int s = 0;
    for (int t = 1; t < ch.nscales; ++t)
        if (block >= (cols ? ch.s[t].col_block0 : ch.s[t].row_block0)) s = t;
    return s;
}

// ------------------------------------------------------------------ row pass

// V4: every scale's rows are whole 16-byte groups (width and plane stride
// multiples of four floats, 16-byte aligned planes), so each lane moves
// four floats per load, store and LDS access (4 loads per image and chunk
// instead of 13); the arithmetic is the same.
template <int NP, bool V4>
__global__ __launch_bounds__(Shape<NP>::kThreads) void ss2_rows(Chain chain, Coef k) {
    constexpr int L = Shape<NP>::kRowLines, NT = Shape<NP>::kThreads, KS = Shape<NP>::kState;
    // chunk columns; tile pitch CH + 4: each lane's row starts 16-byte aligned
    // (so its 64 samples move as 16-byte LDS accesses) and the rows of 16
    // consecutive lanes start 4 banks apart, which keeps those accesses free
    // of bank conflicts
    constexpr int CH = Shape<NP>::kRowChunk, PT = CH + 4;
    constexpr int NI = NP == 1 ? 1 : 2;  // image tiles
    constexpr int RS = NT / CH;      // tile rows one pass of the workgroup covers
    constexpr int KI = (L + RS - 1) / RS;
    constexpr int TILE = L * PT;
    __shared__ __attribute__((aligned(16))) float tin[NI * TILE + PT];  // the image tiles, then a row of ones
    __shared__ __attribute__((aligned(16))) float tout[NP * TILE];

    const int s = scale_of(chain, blockIdx.x, false);
    const ScaleDesc &d = chain.s[s];
    const int local = blockIdx.x - d.row_block0;
    const int c = local % chain.nch, blk = local / chain.nch;
    const int w = d.w, r0 = blk * L, nrows = min(L, d.h - r0);
    const int t = threadIdx.x;
    const int p = t / L, line = t % L;  // this thread's plane and row
    const bool live = p < NP && line < nrows;
    const int nchunks = (w + CH - 1) / CH;
    float *const ck = chain.ckpt + d.ckpt_rows0 + (long long)(blk * chain.nch + c) * nchunks * KS;
    const float *img[2] = {d.a[c], NP == 1 ? d.a[c] : d.b[c]};
    // the plane's factors: a = a 1, b = b 1, a a, b b, a b
    const int f0 = (NP == 5 && (p == 1 || p == 3)) ? 1 : 0;
    const int f1 = (NP == 5 && p >= 3) ? 1 : 0;
    const float *src0 = tin + f0 * TILE + line * PT;
    const float *src1 = (NP == 5 && p >= 2) ? tin + f1 * TILE + line * PT : tin + NI * TILE;
    float *const mine = tout + min(p, NP - 1) * TILE + line * PT;
    const int tcol = t % CH, trow = t / CH;  // tile share (loads and stores)
    constexpr int Q = CH / 4, RS4 = NT / Q, KI4 = (L + RS4 - 1) / RS4;  // the same with float4s
    const int tq = t % Q, trow4 = t / Q;

    if (t < PT) tin[NI * TILE + t] = 1.0f;

    float pre[kRing][NI][KI];
    float4 pre4[kRing][NI][KI4];
    const bool full_rows = nrows == L;
    auto fetch = [&](float (&dst)[NI][KI], int ch) {
        if (ch < 0 || ch >= nchunks) return;
        const int c0 = ch * CH, n = min(CH, w - c0);
        if (full_rows && n == CH) {  // every sample of the tile exists: no per-load guard
#pragma unroll
            for (int q = 0; q < NI; ++q) {
                const float *src = img[q] + (long long)(r0 + trow) * w + c0 + tcol;
#pragma unroll
                for (int i = 0; i < KI; ++i)
                    dst[q][i] = (i < KI - 1 || trow + i * RS < L) ? src[(long long)i * RS * w] : 0.0f;
            }
            return;
        }
#pragma unroll
        for (int q = 0; q < NI; ++q)
#pragma unroll
            for (int i = 0; i < KI; ++i) {
                const int row = trow + i * RS;
                dst[q][i] = (row < nrows && tcol < n) ? img[q][(long long)(r0 + row) * w + c0 + tcol] : 0.0f;
            }
    };
    auto stage = [&](const float (&src)[NI][KI]) {
#pragma unroll
        for (int q = 0; q < NI; ++q)
#pragma unroll
            for (int i = 0; i < KI; ++i) {
                const int row = trow + i * RS;
                if (i < KI - 1 || row < L) tin[q * TILE + row * PT + tcol] = src[q][i];
            }
    };
    // Four columns per lane: a chunk's columns come in whole float4s (the
    // width is a multiple of four), so only rows and whole groups are guarded.
    auto fetch4 = [&](float4 (&dst)[NI][KI4], int ch) {
        if (ch < 0 || ch >= nchunks) return;
        const int c0 = ch * CH, n = min(CH, w - c0);
#pragma unroll
        for (int q = 0; q < NI; ++q) {
            const float *src = img[q] + (long long)(r0 + trow4) * w + c0 + 4 * tq;
#pragma unroll
            for (int i = 0; i < KI4; ++i) {
                const int row = trow4 + i * RS4;
                const bool in = (full_rows && n == CH) ? (i < KI4 - 1 || row < L) : (row < nrows && 4 * tq < n);
                dst[q][i] = in ? *reinterpret_cast<const float4 *>(src + (long long)i * RS4 * w)
                               : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
        }
    };
    auto stage4 = [&](const float4 (&src)[NI][KI4]) {
#pragma unroll
        for (int q = 0; q < NI; ++q)
#pragma unroll
            for (int i = 0; i < KI4; ++i) {
                const int row = trow4 + i * RS4;
                if (i < KI4 - 1 || row < L) *reinterpret_cast<float4 *>(tin + q * TILE + row * PT + 4 * tq) = src[q][i];
            }
    };
    auto samples = [&](float (&v)[CH]) {
#pragma unroll
        for (int j = 0; j < CH; ++j) v[j] = src0[j] * src1[j];
    };

    // Causal walk over every chunk but the last, keeping each end state.
    State f;
    if constexpr (V4) {
        fetch4(pre4[0], 0);
        fetch4(pre4[1], 1);
    } else {
        fetch(pre[0], 0);
        fetch(pre[1], 1);
    }
    auto fbody = [&](auto S, int ch) {
        constexpr int si = decltype(S)::value;
        if (ch >= nchunks - 1) return;
        if constexpr (V4)
            stage4(pre4[si]);
        else
            stage(pre[si]);
        __syncthreads();
        if constexpr (V4)
            fetch4(pre4[(si + 2) % kRing], ch + 2);
        else
            fetch(pre[(si + 2) % kRing], ch + 2);
        if (live) {
            float v[CH];
            samples(v);
            walk_regs<CH, false>(k, v, f);
            ck[ch * KS + t] = f.s1;
            ck[ch * KS + NT + t] = f.s2;
            ck[ch * KS + 2 * NT + t] = f.s3;
        }
        __syncthreads();
    };
    for (int ch = 0; ch < nchunks - 1; ch += kRing) {
        fbody(Ic<0>{}, ch);
        fbody(Ic<1>{}, ch + 1);
        fbody(Ic<2>{}, ch + 2);
    }

    // Anticausal walk, last chunk first: recompute the chunk's causal
    // outputs from the state before it (loaded a chunk ahead), walk back
    // over them, store every plane's chunk row-contiguously.
    State g;
    State before[kRing];
    auto fetch_state = [&](State &dst, int ch) {
        if (ch <= 0) dst = State{};  // the line starts at rest
        if (ch <= 0 || !live) return;
        dst.s1 = ck[(ch - 1) * KS + t];
        dst.s2 = ck[(ch - 1) * KS + NT + t];
        dst.s3 = ck[(ch - 1) * KS + 2 * NT + t];
    };
    if constexpr (V4) {
        fetch4(pre4[0], nchunks - 1);
        fetch4(pre4[1], nchunks - 2);
    } else {
        fetch(pre[0], nchunks - 1);
        fetch(pre[1], nchunks - 2);
    }
    fetch_state(before[0], nchunks - 1);
    auto bbody = [&](auto S, int ch) {
        constexpr int si = decltype(S)::value;
        if (ch < 0) return;
        const int c0 = ch * CH, n = min(CH, w - c0);
        if constexpr (V4)
            stage4(pre4[si]);
        else
            stage(pre[si]);
        __syncthreads();
        if constexpr (V4)
            fetch4(pre4[(si + 2) % kRing], ch - 2);
        else
            fetch(pre[(si + 2) % kRing], ch - 2);
        fetch_state(before[(si + 1) % kRing], ch - 1);
        if (live) {
            State r = before[si];
            if (n == CH) {
                float v[CH];
                samples(v);
                walk_regs<CH, false>(k, v, r);
                walk_regs<CH, true>(k, v, g);
#pragma unroll
                for (int j = 0; j < CH; ++j) mine[j] = v[j];
            } else {  // the row's last chunk: n < 32 samples, walked through LDS
                for (int j = 0; j < n; ++j) mine[j] = r.step(k, src0[j] * src1[j]);
                for (int j = n - 1; j >= 0; --j) mine[j] = g.step(k, mine[j]);
            }
        }
        __syncthreads();
        if constexpr (V4) {  // whole float4 groups: rows and groups past the tile are skipped
#pragma unroll
            for (int q = 0; q < NP; ++q) {
                float *const o = d.rows[c] + (long long)q * d.pstride + (long long)(r0 + trow4) * w + c0 + 4 * tq;
#pragma unroll
                for (int i = 0; i < KI4; ++i) {
                    const int row = trow4 + i * RS4;
                    if (row < nrows && 4 * tq < n)
                        *reinterpret_cast<float4 *>(o + (long long)i * RS4 * w) =
                            *reinterpret_cast<const float4 *>(tout + q * TILE + row * PT + 4 * tq);
                }
            }
        } else if (full_rows && n == CH) {  // every output of the tile exists: unrolled, unguarded but the last row
#pragma unroll
            for (int q = 0; q < NP; ++q) {
                float *const o = d.rows[c] + (long long)q * d.pstride + (long long)(r0 + trow) * w + c0 + tcol;
#pragma unroll
                for (int i = 0; i < KI; ++i)
                    if (i < KI - 1 || trow + i * RS < L)
                        o[(long long)i * RS * w] = tout[q * TILE + (trow + i * RS) * PT + tcol];
            }
        } else if (tcol < n) {
            for (int q = 0; q < NP; ++q) {
                float *const o = d.rows[c] + (long long)q * d.pstride + (long long)r0 * w + c0 + tcol;
                for (int i = trow; i < nrows; i += RS) o[(long long)i * w] = tout[q * TILE + i * PT + tcol];
            }
        }
    };
    for (int ch = nchunks - 1; ch >= 0; ch -= kRing) {
        bbody(Ic<0>{}, ch);
        bbody(Ic<1>{}, ch - 1);
        bbody(Ic<2>{}, ch - 2);
    }
}

// --------------------------------------------------------------- column pass

template <int NP>
__global__ __launch_bounds__(Shape<NP>::kThreads) void ss2_cols(Chain chain, Coef k) {
    constexpr int L = Shape<NP>::kColLines, NT = Shape<NP>::kThreads, KS = Shape<NP>::kState;
    constexpr int CT = kChunk * L;  // pixels of a chunk
    __shared__ float tile[NP * CT];  // [plane][row of the chunk][column]
    __shared__ Pair red[6][NT / 64];

    const int s = scale_of(chain, blockIdx.x, true);
    const ScaleDesc &d = chain.s[s];
    const int local = blockIdx.x - d.col_block0;
    const int c = local % chain.nch, blk = local / chain.nch;
    const int w = d.w, h = d.h, x0 = blk * L, ncols = min(L, w - x0);
    const long long W = w;
    const int t = threadIdx.x;
    const int p = t / L, x = t % L;  // this thread's plane and column
    const bool live = p < NP && x < ncols;
    const float *const col = d.rows[c] + (long long)min(p, NP - 1) * d.pstride + x0 + x;
    float *const ocol = d.out[c] ? d.out[c] + (long long)min(p, NP - 1) * d.pstride + x0 + x : nullptr;
    const int nchunks = (h + kChunk - 1) / kChunk;
    float *const ck = chain.ckpt + d.ckpt_cols0 + (long long)(blk * chain.nch + c) * nchunks * KS;
    const bool stats = chain.partials != nullptr;
    float *const mine = tile + min(p, NP - 1) * CT + x;

    float v[kRing][kChunk];
    auto load = [&](float (&dst)[kChunk], int ch) {
        if (ch < 0 || ch >= nchunks || !live) return;
        const int y0 = ch * kChunk, n = min(kChunk, h - y0);
        const float *src = col + y0 * W;
        if (n == kChunk) {  // no per-load guard
#pragma unroll
            for (int i = 0; i < kChunk; ++i) dst[i] = src[i * W];
            return;
        }
#pragma unroll
        for (int i = 0; i < kChunk; ++i) dst[i] = i < n ? src[i * W] : 0.0f;
    };

    // Causal walk over every chunk but the last, keeping each end state.
    State f;
    load(v[0], 0);
    load(v[1], 1);
    auto fbody = [&](auto S, int ch) {
        constexpr int si = decltype(S)::value;
        if (ch >= nchunks - 1) return;
        load(v[(si + 2) % kRing], ch + 2);
        if (live) {
            walk_regs<kChunk, false>(k, v[si], f);
            ck[ch * KS + t] = f.s1;
            ck[ch * KS + NT + t] = f.s2;
            ck[ch * KS + 2 * NT + t] = f.s3;
        }
    };
    for (int ch = 0; ch < nchunks - 1; ch += kRing) {
        fbody(Ic<0>{}, ch);
        fbody(Ic<1>{}, ch + 1);
        fbody(Ic<2>{}, ch + 2);
    }

    // Anticausal walk, last chunk first; each chunk's five blurred planes
    // then meet in LDS for the statistics of its pixels.
    Acc acc[6];
    State g;
    State before[kRing];
    auto fetch_state = [&](State &dst, int ch) {
        if (ch <= 0) dst = State{};  // the line starts at rest
        if (ch <= 0 || !live) return;
        dst.s1 = ck[(ch - 1) * KS + t];
        dst.s2 = ck[(ch - 1) * KS + NT + t];
        dst.s3 = ck[(ch - 1) * KS + 2 * NT + t];
    };
    // the statistics' image samples of a chunk, thread t taking pixels
    // t, t + NT, ... (row-major over the chunk's 32 x L)
    constexpr int KP = (CT + NT - 1) / NT;
    float ia[KP], ib[KP];
    auto fetch_images = [&](int ch) {
        const int y0 = ch * kChunk, n = min(kChunk, h - y0);
        const float *ra = d.a[c] + (long long)y0 * w + x0, *rb = d.b[c] + (long long)y0 * w + x0;
        const bool full = n == kChunk && ncols == L;
#pragma unroll
        for (int m = 0; m < KP; ++m) {
            const int q = t + m * NT, i = q / L, xx = q % L;
            const bool in = full ? ((m + 1) * NT <= CT || q < CT) : (q < n * L && xx < ncols);
            ia[m] = in ? ra[(long long)i * w + xx] : 0.0f;
            ib[m] = in ? rb[(long long)i * w + xx] : 0.0f;
        }
    };
    load(v[0], nchunks - 1);
    load(v[1], nchunks - 2);
    fetch_state(before[0], nchunks - 1);
    auto bbody = [&](auto S, int ch) {
        constexpr int si = decltype(S)::value;
        if (ch < 0) return;
        const int y0 = ch * kChunk, n = min(kChunk, h - y0);
        load(v[(si + 2) % kRing], ch - 2);
        fetch_state(before[(si + 1) % kRing], ch - 1);
        if (NP == 5 && stats) fetch_images(ch);
        if (live) {
            State r = before[si];
            if (n == kChunk) {
                walk_regs<kChunk, false>(k, v[si], r);
                walk_regs<kChunk, true>(k, v[si], g);
                if (stats) {
#pragma unroll
                    for (int i = 0; i < kChunk; ++i) mine[i * L] = v[si][i];
                }
                if (ocol) {
#pragma unroll
                    for (int i = 0; i < kChunk; ++i) ocol[(y0 + i) * W] = v[si][i];
                }
            } else {  // the column's last chunk: n < 32 rows, walked through LDS
                for (int i = 0; i < n; ++i) mine[i * L] = r.step(k, col[(y0 + i) * W]);
                for (int i = n - 1; i >= 0; --i) {
                    const float y = g.step(k, mine[i * L]);
                    mine[i * L] = y;
                    if (ocol) ocol[(y0 + i) * W] = y;
                }
            }
        }
        if (NP == 5 && stats) {
            __syncthreads();
            // branch-free over the thread's pixels (one basic block, so their
            // long pair-arithmetic chains interleave); a pixel outside the
            // plane enters as zeros, whose terms are exactly 0
#pragma unroll
            for (int m = 0; m < KP; ++m) {
                const int q = t + m * NT, xx = q % L;
                const bool in = q < n * L && xx < ncols;
                const int qq = in ? q : 0;
                pixel_terms(in ? ia[m] : 0.0f, in ? ib[m] : 0.0f, in ? tile[qq] : 0.0f, in ? tile[CT + qq] : 0.0f,
                            in ? tile[2 * CT + qq] : 0.0f, in ? tile[3 * CT + qq] : 0.0f,
                            in ? tile[4 * CT + qq] : 0.0f, acc);
            }
#pragma unroll
            for (int u = 0; u < 6; ++u) acc[u].norm();
            __syncthreads();
        }
    };
    for (int ch = nchunks - 1; ch >= 0; ch -= kRing) {
        bbody(Ic<0>{}, ch);
        bbody(Ic<1>{}, ch - 1);
        bbody(Ic<2>{}, ch - 2);
    }

    if (NP == 5 && stats) {
        Pair sum[6];
#pragma unroll
        for (int m = 0; m < 6; ++m) {
            acc[m].norm();
            sum[m] = Pair{acc[m].hi, acc[m].lo};
        }
        block_pair_sum<NT>(sum, red);
        if (t == 0) {
#pragma unroll
            for (int m = 0; m < 6; ++m) chain.partials[((long long)d.part0 + local) * 6 + m] = sum[m];
        }
    }
}

// One workgroup per (channel, scale): the scale's column-block partials of
// the channel in index order, then the workgroup tree; 6 doubles out.
constexpr int kFinishThreads = 256;

__global__ __launch_bounds__(kFinishThreads) void ss2_chain_finish(Chain chain) {
    __shared__ Pair red[6][kFinishThreads / 64];
    const int c = blockIdx.x, s = blockIdx.y;
    const ScaleDesc &d = chain.s[s];
    const int nblk = (d.w + Shape<5>::kColLines - 1) / Shape<5>::kColLines;
    Pair sum[6];
#pragma unroll
    for (int m = 0; m < 6; ++m) sum[m] = Pair{0.0f, 0.0f};
    for (int blk = threadIdx.x; blk < nblk; blk += kFinishThreads) {
        const long long at = ((long long)d.part0 + (long long)blk * chain.nch + c) * 6;
#pragma unroll
        for (int m = 0; m < 6; ++m) sum[m] = ff_add(sum[m], chain.partials[at + m]);
    }
    block_pair_sum<kFinishThreads>(sum, red);
    if (threadIdx.x == 0) {
        double *r = chain.result + ((long long)s * chain.nch + c) * 6;
#pragma unroll
        for (int m = 0; m < 6; ++m) r[m] = (double)sum[m].hi + (double)sum[m].lo;
        __threadfence_system();
    }
}

// ---------------------------------------------------------------- pyramid

// Every later scale of the pyramid in one launch.  A workgroup owns a
// 64 x 64 tile of the first scale: its 32 x 32 downsample, that tile's
// 16 x 16 downsample and so on are tiles of the later scales, aligned on
// their own edges, so the pixels a later scale's pixel averages (the
// replicated last column or row included: it is the pixel just before,
// inside the same tile) stay in the workgroup, and the scales after the
// second are formed from LDS.  Each scale's pixel is
// ((a + b) + (c + d)) * 0.25f over its 2 x 2 block, a and b from the upper
// row, the last column and row repeated when the size is odd.
constexpr int kPyrEdge = 32;  // a workgroup's tile edge at the second scale

struct PyrPass {
    const float *in[2 * kSs2MaxChannels];
    float *out[kSs2MaxScales - 1][2 * kSs2MaxChannels];
    int w[kSs2MaxScales], h[kSs2MaxScales];
    int levels, tiles_x;
};

__device__ inline float mean4(float a, float b, float c, float d) { return ((a + b) + (c + d)) * 0.25f; }

// Scale L (2..5) of the tile from scale L-1's tile in LDS (pitch 2E+1).
template <int L>
__device__ void pyramid_level(const PyrPass &p, int plane, int tx, int ty, const float *src, float *dst) {
    constexpr int E = kPyrEdge >> (L - 1);  // this scale's tile edge
    constexpr int SP = 2 * E + 1, DP = E + 1;
    const int t = threadIdx.x;
    if (t >= E * E) return;
    const int r = t / E, c = t % E;
    const int y = ty * E + r, x = tx * E + c;
    const int ow = p.w[L], oh = p.h[L], pw = p.w[L - 1], ph = p.h[L - 1];
    if (y >= oh || x >= ow) return;
    const int r0 = 2 * r, r1 = min(2 * y + 1, ph - 1) - 2 * E * ty;
    const int c0 = 2 * c, c1 = min(2 * x + 1, pw - 1) - 2 * E * tx;
    const float v = mean4(src[r0 * SP + c0], src[r0 * SP + c1], src[r1 * SP + c0], src[r1 * SP + c1]);
    if (dst) dst[r * DP + c] = v;
    p.out[L - 1][plane][(long long)y * ow + x] = v;
}

__global__ __launch_bounds__(256) void ss2_pyramid(PyrPass p) {
    __shared__ float t1[32 * 33], t2[16 * 17], t3[8 * 9], t4[4 * 5];
    const int plane = blockIdx.y;
    const int tx = blockIdx.x % p.tiles_x, ty = blockIdx.x / p.tiles_x;
    {  // the second scale from the caller's plane: four pixels per thread,
       // every load issued before any sum (the loads of pixels outside the
       // plane are clamped in, their results dropped)
        const float *in = p.in[plane];
        const int w = p.w[0], h = p.h[0], ow = p.w[1], oh = p.h[1];
        float q[4][4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = threadIdx.x + 256 * k;
            const int y = min(ty * kPyrEdge + (i >> 5), oh - 1), x = min(tx * kPyrEdge + (i & 31), ow - 1);
            const long long r0 = (long long)(2 * y) * w, r1 = (long long)min(2 * y + 1, h - 1) * w;
            const int c0 = 2 * x, c1 = min(2 * x + 1, w - 1);
            q[k][0] = in[r0 + c0];
            q[k][1] = in[r0 + c1];
            q[k][2] = in[r1 + c0];
            q[k][3] = in[r1 + c1];
        }
        float *out = p.out[0][plane];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = threadIdx.x + 256 * k;
            const int r = i >> 5, c = i & 31;
            const int y = ty * kPyrEdge + r, x = tx * kPyrEdge + c;
            if (y < oh && x < ow) {
                const float v = mean4(q[k][0], q[k][1], q[k][2], q[k][3]);
                t1[r * 33 + c] = v;
                out[(long long)y * ow + x] = v;
            }
        }
    }
    if (p.levels < 2) return;
    __syncthreads();
    pyramid_level<2>(p, plane, tx, ty, t1, t2);
    if (p.levels < 3) return;
    __syncthreads();
    pyramid_level<3>(p, plane, tx, ty, t2, t3);
    if (p.levels < 4) return;
    __syncthreads();
    pyramid_level<4>(p, plane, tx, ty, t3, t4);
    if (p.levels < 5) return;
    __syncthreads();
    pyramid_level<5>(p, plane, tx, ty, t4, nullptr);
}

template <int NP>
int row_blocks(int h) {
    return (h + Shape<NP>::kRowLines - 1) / Shape<NP>::kRowLines;
}
template <int NP>
int col_blocks(int w) {
    return (w + Shape<NP>::kColLines - 1) / Shape<NP>::kColLines;
}
template <int NP>
long long rows_ckpt(int w, int h) {
    return (long long)row_blocks<NP>(h) * ((w + Shape<NP>::kRowChunk - 1) / Shape<NP>::kRowChunk) *
           Shape<NP>::kState;
}
template <int NP>
long long cols_ckpt(int w, int h) {
    return (long long)col_blocks<NP>(w) * ((h + kChunk - 1) / kChunk) * Shape<NP>::kState;
}

// Fills the per-scale offsets; returns the checkpoint floats and partials
// the chain needs.
template <int NP>
void plan(Chain &ch, long long *ckpt_floats, long long *partials) {
    int rb = 0, cb = 0, part = 0;
    long long ckr = 0, ckc = 0;
    for (int s = 0; s < ch.nscales; ++s) {
        ScaleDesc &d = ch.s[s];
        d.row_block0 = rb;
        d.col_block0 = cb;
        d.ckpt_rows0 = ckr;
        d.ckpt_cols0 = ckc;
        d.part0 = part;
        rb += row_blocks<NP>(d.h) * ch.nch;
        cb += col_blocks<NP>(d.w) * ch.nch;
        ckr += rows_ckpt<NP>(d.w, d.h) * ch.nch;
        ckc += cols_ckpt<NP>(d.w, d.h) * ch.nch;
        part += col_blocks<NP>(d.w) * ch.nch;
    }
    *ckpt_floats = std::max(ckr, ckc);  // the row pass's checkpoints are dead once the column pass runs
    *partials = part;
}

}  // namespace

size_t ss2_chain_scratch_floats(int nch, int nplanes, const int *w, const int *h, int nscales) {
    Chain ch{};
    ch.nch = nch;
    ch.nscales = nscales;
    for (int s = 0; s < nscales; ++s) {
        ch.s[s].w = w[s];
        ch.s[s].h = h[s];
    }
    long long ck = 0, part = 0;
    if (nplanes == 5)
        plan<5>(ch, &ck, &part);
    else
        plan<1>(ch, &ck, &part);
    return (size_t)ck + (size_t)part * 6 * 2;
}

hipError_t launch_ss2_chain(const Ss2ChainArgs &args, hipStream_t stream, const KernelTimer &rows_timer,
                            const KernelTimer &cols_timer) {
    const int np = args.nplanes, nch = args.nch, ns = args.nscales;
    if (nch < 1 || nch > kSs2MaxChannels || ns < 1 || ns > kSs2MaxScales || (np != 1 && np != 5) || !args.scratch)
        return hipErrorInvalidValue;
    if (np == 1 && (nch != 1 || args.stats)) return hipErrorInvalidValue;
    if (np == 5 && !args.stats) return hipErrorInvalidValue;  // the five-plane column pass always sums
    if (args.stats && !args.result) return hipErrorInvalidValue;
    Chain ch{};
    ch.nch = nch;
    ch.nscales = ns;
    for (int s = 0; s < ns; ++s) {
        const Ss2Scale &in = args.scale[s];
        ScaleDesc &d = ch.s[s];
        if (in.w < 1 || in.h < 1) return hipErrorInvalidValue;
        d.w = in.w;
        d.h = in.h;
        d.pstride = in.pstride;
        for (int c = 0; c < nch; ++c) {
            d.a[c] = in.a[c];
            d.b[c] = np == 5 ? in.b[c] : in.a[c];
            d.rows[c] = in.rows[c];
            d.out[c] = in.out[c];
        }
    }
    long long ck = 0, part = 0;
    if (np == 5)
        plan<5>(ch, &ck, &part);
    else
        plan<1>(ch, &ck, &part);
    ch.ckpt = args.scratch;
    ch.partials = args.stats ? reinterpret_cast<Pair *>(args.scratch + ck) : nullptr;
    ch.result = args.result;
    const Coef k{args.coef[0], args.coef[1], args.coef[2], args.coef[3]};
    const ScaleDesc &last = ch.s[ns - 1];
    const int nrow = last.row_block0 + (np == 5 ? row_blocks<5>(last.h) : row_blocks<1>(last.h)) * nch;
    const int ncol = last.col_block0 + (np == 5 ? col_blocks<5>(last.w) : col_blocks<1>(last.w)) * nch;
    hipError_t e;
    // Whole 16-byte groups at every scale: widths and plane strides multiples
    // of four floats, images and row planes 16-byte aligned.
    bool v4 = true;
    for (int s = 0; s < ns; ++s) {
        const ScaleDesc &d = ch.s[s];
        v4 = v4 && d.w % 4 == 0 && d.pstride % 4 == 0;
        for (int c = 0; c < nch; ++c)
            v4 = v4 && ((reinterpret_cast<uintptr_t>(d.a[c]) | reinterpret_cast<uintptr_t>(d.b[c]) |
                         reinterpret_cast<uintptr_t>(d.rows[c])) & 15u) == 0;
    }
    if (np == 5) {
        e = v4 ? launch_kernel(ss2_rows<5, true>, dim3(nrow), dim3(Shape<5>::kThreads), stream, rows_timer, ch, k)
               : launch_kernel(ss2_rows<5, false>, dim3(nrow), dim3(Shape<5>::kThreads), stream, rows_timer, ch, k);
        if (e == hipSuccess)
            e = launch_kernel(ss2_cols<5>, dim3(ncol), dim3(Shape<5>::kThreads), stream, cols_timer, ch, k);
    } else {
        e = launch_kernel(ss2_rows<1, false>, dim3(nrow), dim3(Shape<1>::kThreads), stream, rows_timer, ch, k);
        if (e == hipSuccess)
            e = launch_kernel(ss2_cols<1>, dim3(ncol), dim3(Shape<1>::kThreads), stream, cols_timer, ch, k);
    }
    if (e != hipSuccess || !args.stats) return e;
    hipLaunchKernelGGL(ss2_chain_finish, dim3(nch, ns), dim3(kFinishThreads), 0, stream, ch);
    return hipGetLastError();
}

void ss2_downsampled_dim(int w, int h, int *ow, int *oh) {
    *ow = (w + 1) / 2;
    *oh = (h + 1) / 2;
}

hipError_t launch_ss2_pyramid(const float *const *in, float *const *out, int nplanes, int w, int h, int levels,
                              hipStream_t stream) {
    if (nplanes < 1 || nplanes > 2 * kSs2MaxChannels || w < 1 || h < 1 || levels < 1 || levels > kSs2MaxScales - 1)
        return hipErrorInvalidValue;
    PyrPass p{};
    p.w[0] = w;
    p.h[0] = h;
    for (int l = 1; l <= levels; ++l) ss2_downsampled_dim(p.w[l - 1], p.h[l - 1], &p.w[l], &p.h[l]);
    for (int i = 0; i < nplanes; ++i) {
        p.in[i] = in[i];
        for (int l = 0; l < levels; ++l) p.out[l][i] = out[l * nplanes + i];
    }
    p.levels = levels;
    p.tiles_x = (p.w[1] + kPyrEdge - 1) / kPyrEdge;
    const long long tiles = (long long)p.tiles_x * ((p.h[1] + kPyrEdge - 1) / kPyrEdge);
    hipLaunchKernelGGL(ss2_pyramid, dim3((unsigned)tiles, nplanes), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace vqm
