// ssim_step.hip — the float_ssim step kernel: decimation, SSIM map and
// fixed-tree reduction of a stream of frame batches, software-pipelined.
//
// "ADR-1405: float_ssim_hip decimates on the device, bit-identical to the
// CPU", Context and Decision 1–4: each plane is decimated (exactly, see
// decimate_device.h), then the 11x11 Gaussian local means, variances and
// covariance give a per-pixel SSIM term over the valid region whose mean is
// the frame score; at scale 1 the map reads the raw samples directly.
// "Research-1363: Device-resident ssimulacra2 and a single-wait MS-SSIM on
// SYCL", Finding 4: the sum runs through a fixed tree — a fixed pixel subset
// per work-item, a tree per work-group, one group over the partials — so
// the result depends only on the plane size.
//
// One launch holds three independent roles, each over its own batch of
// frames: decimation of batch k, the SSIM map of batch k-1 (whose decimated
// planes the previous launch wrote) and the finish of batch k-2 (whose
// partials the previous launch wrote).  No workgroup waits for another, and
// the map's ALU work overlaps the decimation's HBM streaming inside one grid
// instead of costing a launch of its own.  Every XCD receives, in order, its
// map workgroups, its eighth of the decimation workgroups and its share of
// the finish workgroups (StepLayout).
//
// Map role: a workgroup scores TW x TH tiles of the map one after another.
// A tile's (TW+10) x (TH+10) input window of both planes is staged in LDS, the
// horizontal 11-tap pass writes four moment planes over it (x, y, x^2 + y^2
// and xy: the map needs the two variances only as their sum; four columns per
// thread step), and the vertical pass (four rows per thread step) forms the
// moments of each map pixel and its SSIM term in fp32, with the mid-scale
// offset removed first so E[x^2] - mu^2 cancels less.  Each thread adds its
// map pixels in fp64 and the workgroup's fixed-tree sum goes to the
// frame's partials array.  Finish role: one workgroup per frame sums the
// partials in index order and writes the mean straight into the pinned host
// result slot.
#include "decimate_device.h"
#include "ssim_common.h"

#include <type_traits>

namespace vqm {
namespace {

constexpr int kNT = 256;                       // threads per workgroup, every role
constexpr int kTW = 32, kTH = 32, kRB = 4;     // map tile
constexpr int kNP = 4;                         // moment planes: x, y, x^2 + y^2, xy
constexpr int kDecWaves = kNT / 64;            // waves per decimation workgroup

// ------------------------------------------------------------ decimation policies

// Each policy's run() gets the workgroup's LDS buffer (the map tile's, which
// a workgroup of the decimation role does not otherwise use).
struct DecNone {
    static constexpr bool kStreams = false;  // whether the decimation is the wide HBM stream (see map_tile)
    static int blocks_per_frame(const StepGeometry &) { return 0; }
    __device__ static void run(const DecimateFrame &, int, const StepGeometry &, float *) {}
};

template <typename T, int S>
struct DecPow2 {
    static constexpr bool kStreams = true;
    using Sh = dec::Pow2Shape<T, S>;
    __host__ __device__ static int waves_per_row(const StepGeometry &g) {
        const int groups = (g.dec_w + Sh::CPT - 1) / Sh::CPT;  // groups holding outputs
        return (groups + 62) / 63;
    }
    // Units (row, wave-in-row) a wave takes in turn: two where a row needs
    // at most two waves (1080p), so that fewer, longer decimation workgroups
    // leave the interleaved map tiles more of the CUs (1080p step 43.0 ->
    // 39.1 us per launch of 32 frames; loading both units before adding
    // either measured no faster, 39.4 -> 39.5 us, and its registers cost the
    // 2160p step 177.7 -> 180.2 us); one on wide rows, where the decimation
    // is the HBM stream and a second unit per wave only delays it (2160p
    // 179.8 -> 196.5 us).
    __host__ __device__ static int units_per_wave(const StepGeometry &g) { return waves_per_row(g) <= 2 ? 2 : 1; }
    // A frame's units in row order, units_per_wave to a wave and kDecWaves
    // waves to a workgroup, so rows that need fewer waves than a workgroup
    // has leave no wave idle.
    static int blocks_per_frame(const StepGeometry &g) {
        const int upw = units_per_wave(g);
        const int waves = (waves_per_row(g) * g.dec_h + upw - 1) / upw;
        return (waves + kDecWaves - 1) / kDecWaves;
    }
    __device__ static void run(const DecimateFrame &fr, int b, const StepGeometry &g, float *) {
        const int wpr = waves_per_row(g), upw = units_per_wave(g);
        const int u0 = (b * kDecWaves + (int)(threadIdx.x >> 6)) * upw;
#pragma unroll 1
        for (int u = u0; u < u0 + upw; ++u) {
            if (u >= wpr * g.dec_h) return;  // the frame's last workgroup may be partly empty
            const int Y = u / wpr;
            dec::pow2_wave<T, S>(fr, u - Y * wpr, Y, g.w, g.h, g.dec_w, g.post, g.dec_pitch, g.packed != 0);
        }
    }
};

// Any other scale: one workgroup per (output row, segment of windows).
template <typename T>
struct DecGeneral {
    static constexpr bool kStreams = false;
    __host__ __device__ static int segments(const StepGeometry &g) {
        const int k = dec::gen_windows_per_block(g.s);
        return (g.dec_w + k - 1) / k;
    }
    static int blocks_per_frame(const StepGeometry &g) { return segments(g) * g.dec_h; }
    __device__ static void run(const DecimateFrame &fr, int b, const StepGeometry &g, float *smem) {
        const int segs = segments(g);
        const int Y = b / segs;
        dec::general_rows_block<T>(fr, b - Y * segs, Y, g.w, g.h, g.bpc, g.s, g.tap, g.dec_w, g.dec_pitch,
                                   g.packed != 0, reinterpret_cast<int *>(smem));
    }
};

// s = 2^k on planes the vector path cannot take (rows not 16-byte aligned).
template <typename T, int S>
struct DecPow2Scalar {
    static constexpr bool kStreams = false;
    __host__ __device__ static int blocks_x(const StepGeometry &g) { return (g.dec_w + 63) / 64; }
    static int blocks_per_frame(const StepGeometry &g) {
        constexpr int rows = 4 * dec::scalar_rows_per_thread<S>();  // output rows per workgroup
        return blocks_x(g) * ((g.dec_h + rows - 1) / rows);
    }
    __device__ static void run(const DecimateFrame &fr, int b, const StepGeometry &g, float *) {
        const int bx = b % blocks_x(g), by = b / blocks_x(g);
        dec::pow2_scalar_block<T, S>(fr, bx, by, g.w, g.h, g.dec_w, g.dec_h, g.dec_pitch, g.post, g.packed != 0);
    }
};

// ------------------------------------------------------------ map and finish roles

__host__ __device__ inline int tiles_x(const StepGeometry &g) { return (g.dec_w - 10 + kTW - 1) / kTW; }
__host__ __device__ inline int tiles_y(const StepGeometry &g) { return (g.dec_h - 10 + kTH - 1) / kTH; }

// In the looping layout (below) with the vector decimation the tile buffer is
// oversized on purpose: LDS (160 KiB per CU) is what limits how many step
// workgroups share a CU, and at 2160p that decimation streams fastest with at
// most three of them per CU.  The scalar and general decimations are bound by
// load latency instead and keep every slot.
// Measured per launch of 32 frames: 198.3 us with two, 189.1 us with three,
// 190.9 us with four, 192.1 us with no cap (VGPRs then allow four).
constexpr int kLoopWorkgroupsPerCu = 3;
constexpr int kLoopLdsFloats = (160 * 1024 / (kLoopWorkgroupsPerCu + 1)) / 4;
static_assert(kLoopLdsFloats >= tile_lds_floats<kTW, kTH, kNP>(), "the capped tile buffer must hold the tile");
static_assert(kLoopWorkgroupsPerCu * (kLoopLdsFloats * 4 + 1024) <= 160 * 1024,
              "the capped buffer must still let kLoopWorkgroupsPerCu workgroups share a CU");

// LDS floats of a step workgroup: the map tile's buffer (oversized on
// purpose in the capped layout), which the general decimation borrows.
template <bool kCapped>
constexpr int step_lds_floats() {
    return kCapped ? kLoopLdsFloats : tile_lds_floats<kTW, kTH, kNP>();
}
static_assert(tile_lds_floats<kTW, kTH, kNP>() >= dec::kGenLdsInts, "the general decimation borrows the tile buffer");

template <typename TIn>
__device__ __forceinline__ void map_tile(const SsimFrame &fr, int tile, const StepGeometry &g, int pitch,
                                         float unit, bool vec4, const Taps &taps, float *lds) {
    constexpr int IH = kTH + 10, IP = in_pitch<kTW>();
    __shared__ double red[1][kNT / 64];
    float *sx = lds, *sy = lds + IH * IP;

    const int tx = tiles_x(g);
    const int bx = tile % tx, by = tile / tx;
    const TIn *ref = static_cast<const TIn *>(fr.ref);
    const TIn *dis = static_cast<const TIn *>(fr.dis);
    const int W = g.dec_w, H = g.dec_h, MW = W - 10, MH = H - 10;
    const int x0 = bx * kTW, y0 = by * kTH;

    stage<kTW, kTH, kNT>(ref, dis, pitch, W, H, unit, x0, y0, sx, sy, vec4);
    __syncthreads();
    horizontal_moments_in_place<kTW, kTH, kNT, kNP>(lds, taps);

    // A thread's few map pixels and then its wave are summed in fp32, the
    // waves in fp64.
    float part = 0.0f;
    vertical_moments<kTW, kTH, kNT, kRB, kNP>(lds, taps, x0, y0, MW, MH,
                                              [&](int, int, const float (&m)[kNP]) {
        part += ssim_term4(m[0], m[1], m[2], m[3]);
    });

    const float terms[1] = {part};
    double acc[1];
    block_sum_terms<kNT, 1>(terms, red, acc);
    if (threadIdx.x == 0) fr.partials[tile] = acc[0];
}

// The frame's score goes to result[0]; result[1] receives the decibel form
// only when the caller asked for it, so the read-back is 8 bytes otherwise.
__device__ __forceinline__ void finish_frame(const SsimFrame &fr, const StepGeometry &g, bool want_db) {
    __shared__ double red[1][kNT / 64];
    double tot[1];
    sum_spans<kNT, 1>(fr.partials, tiles_x(g) * tiles_y(g), 0, tot, red);
    if (threadIdx.x == 0) {
        const double m = tot[0] / ((double)(g.dec_w - 10) * (double)(g.dec_h - 10));
        fr.result[0] = m;
        // The decibel form -10 log10(1 - ssim), +inf for a score of 1 or
        // more ("ADR-1405: float_ssim_hip decimates on the device,
        // bit-identical to the CPU", Consequences: enable_db).
        if (want_db) fr.result[1] = m < 1.0 ? -10.0 * log10(1.0 - m) : (m >= 1.0 ? __builtin_inf() : m);
        __threadfence_system();
    }
}

// Where each role sits in the grid.  The dispatcher hands workgroup L to
// XCD L % 8; position q = L / 8 is the order in which that XCD receives its
// workgroups.  Each XCD gets, in order: its map workgroups (over its eighth
// of the map tiles), then its eighth of the decimation workgroups
// (short-lived, so the dispatcher balances them), then its share of the
// finish workgroups.
//
// Three shapes of the map role.  When the decimation streams far more bytes
// than the map has tiles (2160p: ~270 KB of raw input per map tile), ~32 map
// workgroups per XCD loop over the tiles: the map holds about one slot per
// CU for the whole launch and hides under the decimation, which keeps the
// other slots.  Otherwise every tile gets its own workgroup, so the map runs
// at full width: interleaved with the decimation workgroups when the
// decimation still reads enough per tile to take about as long (1080p: ~31 KB
// per tile), ahead of them when the map dominates (853x481: ~15 KB).
// Measured at 8 frames per launch: 2160p 47.8 us looping against 49.7 us
// one tile each; 1080p 21.1 us looping against 15.6 us one tile each.
struct StepLayout {
    int map_per_xcd;   // map tiles per XCD (contiguous ranges of the tile order)
    int map_wg;        // map workgroups per XCD
    int dec_per_xcd;   // decimation workgroups per XCD
    int fin_per_xcd;   // finish workgroups per XCD
    int interleave;    // 1: one tile per map workgroup, interleaved with the decimation workgroups
};

// Map workgroups per XCD when they loop: about one per CU.
constexpr int kMapWorkgroupsPerXcd = 32;
// Raw input bytes the decimation reads per map tile above which the map
// workgroups loop.
constexpr long long kLoopBytesPerTile = 100 * 1024;
// Below that, and above this, one-tile map workgroups are interleaved with
// the decimation workgroups instead of dispatched ahead of them: the
// decimation's HBM time is then about the map's ALU time or more, and both
// run side by side.  Measured per launch of 32 frames: 1080p (31 KB per
// tile) 45.1 us ahead, 42.9 us interleaved; 853x481 (15 KB per tile, the
// map dominates and its long tiles are best started first) 39.8 us ahead,
// 43.0 us interleaved.
constexpr long long kInterleaveBytesPerTile = 20 * 1024;

template <class Dec, typename TIn, bool kLoopMap>
__global__ __launch_bounds__(kNT) void ssim_step(StepRoles r, StepGeometry g, StepLayout lay, int map_pitch,
                                                 float unit, int vec4, Taps taps) {
    __shared__ __attribute__((aligned(16))) float smem[step_lds_floats<kLoopMap && Dec::kStreams>()];
    const int x = (int)(blockIdx.x & 7u);
    int q = (int)(blockIdx.x >> 3);
    if (!kLoopMap && lay.interleave) {
        // Position q of this XCD's map_wg + dec_per_xcd first workgroups is a
        // map workgroup when floor((q+1) M / (M+D)) > floor(q M / (M+D)): the
        // map's M tiles spread evenly among the D decimation workgroups, so
        // that ALU-bound map tiles and HBM-bound decimation share the CUs.
        const int M = lay.map_wg, MD = lay.map_wg + lay.dec_per_xcd;
        if (q < MD) {
            const int mq = (int)((long long)q * M / MD), mq1 = (int)((long long)(q + 1) * M / MD);
            if (mq1 > mq) {
                const int map_pf = tiles_x(g) * tiles_y(g);
                const int m = x * lay.map_per_xcd + mq;
                if (mq < lay.map_per_xcd && m < r.n_map * map_pf) {
                    const int f = m / map_pf;
                    map_tile<TIn>(r.map.f[f], m - f * map_pf, g, map_pitch, unit, vec4 != 0, taps, smem);
                }
                return;
            }
            const int dec_pf = r.dec_blocks_per_frame;
            const int d = x * lay.dec_per_xcd + (q - mq);
            if (d < r.n_dec * dec_pf) {
                const int f = d / dec_pf;
                Dec::run(r.dec.f[f], d - f * dec_pf, g, smem);
            }
            return;
        }
        q -= MD;
        const int fi = x * lay.fin_per_xcd + q;
        if (fi < r.n_fin) finish_frame(r.fin.f[fi], g, (r.fin_db_mask >> fi) & 1u);
        return;
    }
    if (q < lay.map_wg) {
        const int map_pf = tiles_x(g) * tiles_y(g);
        const int m0 = x * lay.map_per_xcd;
        const int m1 = min(m0 + lay.map_per_xcd, r.n_map * map_pf);
        if constexpr (kLoopMap) {
#pragma unroll 1
            for (int m = m0 + q; m < m1; m += lay.map_wg) {
                const int f = m / map_pf;
                map_tile<TIn>(r.map.f[f], m - f * map_pf, g, map_pitch, unit, vec4 != 0, taps, smem);
                __syncthreads();  // the next tile reuses the LDS
            }
        } else {
            const int m = m0 + q;
            if (m < m1) {
                const int f = m / map_pf;
                map_tile<TIn>(r.map.f[f], m - f * map_pf, g, map_pitch, unit, vec4 != 0, taps, smem);
            }
        }
        return;
    }
    q -= lay.map_wg;
    if (q < lay.dec_per_xcd) {
        const int dec_pf = r.dec_blocks_per_frame;
        const int d = x * lay.dec_per_xcd + q;
        if (d < r.n_dec * dec_pf) {
            const int f = d / dec_pf;
            Dec::run(r.dec.f[f], d - f * dec_pf, g, smem);
        }
        return;
    }
    q -= lay.dec_per_xcd;
    const int fi = x * lay.fin_per_xcd + q;
    if (fi < r.n_fin) finish_frame(r.fin.f[fi], g, (r.fin_db_mask >> fi) & 1u);
}

template <class Dec, typename TIn>
hipError_t launch_step(StepRoles r, const StepGeometry &g, int map_pitch, float unit, const Taps &taps,
                       hipStream_t stream, const KernelTimer &timer) {
    r.dec_blocks_per_frame = r.n_dec > 0 ? Dec::blocks_per_frame(g) : 0;
    if (r.n_dec > 0 && r.dec_blocks_per_frame == 0) return hipErrorInvalidValue;
    const long long dec_blocks = (long long)r.n_dec * r.dec_blocks_per_frame;
    const long long map_tiles = (long long)r.n_map * tiles_x(g) * tiles_y(g);
    if (dec_blocks > 0x0fffffffLL || map_tiles > 0x0fffffffLL) return hipErrorInvalidValue;
    const long long raw_bytes = 2LL * r.n_dec * g.w * g.h * (g.bpc == 8 ? 1 : 2);
    const bool loop = map_tiles > 0 && raw_bytes >= kLoopBytesPerTile * map_tiles;
    StepLayout lay;
    lay.map_per_xcd = (int)((map_tiles + 7) / 8);
    lay.map_wg = loop ? min(kMapWorkgroupsPerXcd, lay.map_per_xcd) : lay.map_per_xcd;
    lay.dec_per_xcd = (int)((dec_blocks + 7) / 8);
    lay.fin_per_xcd = (r.n_fin + 7) / 8;
    lay.interleave = !loop && map_tiles > 0 && dec_blocks > 0 && raw_bytes >= kInterleaveBytesPerTile * map_tiles;
    const long long blocks = 8LL * (lay.map_wg + lay.dec_per_xcd + lay.fin_per_xcd);
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    int vec4 = 1;
    for (int i = 0; i < r.n_map; ++i)
        if (!stage_vec4_ok(r.map.f[i].ref, map_pitch, sizeof(TIn)) ||
            !stage_vec4_ok(r.map.f[i].dis, map_pitch, sizeof(TIn)))
            vec4 = 0;
    if constexpr (!std::is_same<Dec, DecNone>::value) {
        if (loop)
            return launch_kernel(ssim_step<Dec, TIn, true>, dim3((unsigned)blocks), dim3(kNT), stream, timer, r, g,
                                 lay, map_pitch, unit, vec4, taps);
    }
    return launch_kernel(ssim_step<Dec, TIn, false>, dim3((unsigned)blocks), dim3(kNT), stream, timer, r, g, lay,
                         map_pitch, unit, vec4, taps);
}

template <typename T, typename TIn>
hipError_t launch_dec_pow2(int s, const StepRoles &r, const StepGeometry &g, int map_pitch, float unit,
                           const Taps &taps, hipStream_t stream, const KernelTimer &timer) {
    switch (s) {
    case 2: return launch_step<DecPow2<T, 2>, TIn>(r, g, map_pitch, unit, taps, stream, timer);
    case 4: return launch_step<DecPow2<T, 4>, TIn>(r, g, map_pitch, unit, taps, stream, timer);
    case 8: return launch_step<DecPow2<T, 8>, TIn>(r, g, map_pitch, unit, taps, stream, timer);
    case 16: return launch_step<DecPow2<T, 16>, TIn>(r, g, map_pitch, unit, taps, stream, timer);
    case 32: return launch_step<DecPow2<T, 32>, TIn>(r, g, map_pitch, unit, taps, stream, timer);
    case 64: return launch_step<DecPow2<T, 64>, TIn>(r, g, map_pitch, unit, taps, stream, timer);
    case 128: return launch_step<DecPow2<T, 128>, TIn>(r, g, map_pitch, unit, taps, stream, timer);
    default: return hipErrorInvalidValue;
    }
}

// s = 2^k on rows that are not 16-byte aligned: the scalar integer path.
template <typename T, typename TIn>
hipError_t launch_dec_pow2_scalar(int s, const StepRoles &r, const StepGeometry &g, int map_pitch, float unit,
                                  const Taps &taps, hipStream_t stream, const KernelTimer &timer) {
    switch (s) {
    case 2: return launch_step<DecPow2Scalar<T, 2>, TIn>(r, g, map_pitch, unit, taps, stream, timer);
    case 4: return launch_step<DecPow2Scalar<T, 4>, TIn>(r, g, map_pitch, unit, taps, stream, timer);
    case 8: return launch_step<DecPow2Scalar<T, 8>, TIn>(r, g, map_pitch, unit, taps, stream, timer);
    case 16: return launch_step<DecPow2Scalar<T, 16>, TIn>(r, g, map_pitch, unit, taps, stream, timer);
    default: return launch_step<DecGeneral<T>, TIn>(r, g, map_pitch, unit, taps, stream, timer);
    }
}

// The packed scales: s = 2^k with bpc + 2k <= 16, so s <= 16 for 8-bit and
// s <= 8 for deeper samples; the map reads the uint16 window sums.
template <typename T>
hipError_t launch_dec_pow2_packed(int s, const StepRoles &r, const StepGeometry &g, int map_pitch, float unit,
                                  const Taps &taps, hipStream_t stream, const KernelTimer &timer) {
    switch (s) {
    case 2: return launch_step<DecPow2<T, 2>, uint16_t>(r, g, map_pitch, unit, taps, stream, timer);
    case 4: return launch_step<DecPow2<T, 4>, uint16_t>(r, g, map_pitch, unit, taps, stream, timer);
    case 8: return launch_step<DecPow2<T, 8>, uint16_t>(r, g, map_pitch, unit, taps, stream, timer);
    case 16:
        if constexpr (sizeof(T) == 1) return launch_step<DecPow2<T, 16>, uint16_t>(r, g, map_pitch, unit, taps,
                                                                                 stream, timer);
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool decimate_fast_path(const DecimateBatch &b, int n, int w, int h, int bpc, int s) {
    (void)h;
    if (s < 2 || s > 128 || (s & (s - 1)) != 0) return false;
    const int V = bpc == 8 ? 16 : 8;
    if (w % V != 0) return false;
    for (int i = 0; i < n; ++i)
        if (((uintptr_t)b.f[i].ref | (uintptr_t)b.f[i].dis) & 15u) return false;
    const int dec_w = (w + s - 1) / s;
    // the last window's right half must lie inside the row (no right mirror)
    if (w - s * (dec_w - 1) < s / 2) return false;
    return true;
}

int ssim_partials(int W, int H) {
    return ((W - 10 + kTW - 1) / kTW) * ((H - 10 + kTH - 1) / kTH);
}

hipError_t launch_ssim_step(const StepRoles &r, const StepGeometry &g, InKind map_kind, int map_pitch, float unit,
                            const Taps &taps, hipStream_t stream, const KernelTimer &timer) {
    if (r.n_dec < 0 || r.n_dec > kMaxBatch || r.n_map < 0 || r.n_map > kMaxBatch || r.n_fin < 0 ||
        r.n_fin > kMaxBatch)
        return hipErrorInvalidValue;
    if ((g.packed != 0) != packed_planes(g.s, g.bpc)) return hipErrorInvalidValue;
    if (r.n_dec > 0) {
        // The map role reads what the decimation writes: uint16 window sums
        // or fp32 values.
        if (map_kind != (g.packed ? IN_U16 : IN_F32) && r.n_map > 0) return hipErrorInvalidValue;
        // The vector path stores a lane's outputs as one 16-byte (or smaller)
        // group: planes 16-byte aligned, pitch a multiple of 8 outputs (the
        // library's planes are 256-byte aligned with a pitch of 64 k).
        bool out_aligned = g.dec_pitch % 8 == 0;
        for (int i = 0; i < r.n_dec; ++i)
            if (((uintptr_t)r.dec.f[i].out_ref | (uintptr_t)r.dec.f[i].out_dis) & 15u) out_aligned = false;
        const bool fast = out_aligned && decimate_fast_path(r.dec, r.n_dec, g.w, g.h, g.bpc, g.s);
        if (g.packed) {
            // packed implies s = 2^k: the vector path, else the scalar one
            if (g.bpc == 8) {
                if (fast) return launch_dec_pow2_packed<uint8_t>(g.s, r, g, map_pitch, unit, taps, stream, timer);
                return launch_dec_pow2_scalar<uint8_t, uint16_t>(g.s, r, g, map_pitch, unit, taps, stream, timer);
            }
            if (fast) return launch_dec_pow2_packed<uint16_t>(g.s, r, g, map_pitch, unit, taps, stream, timer);
            return launch_dec_pow2_scalar<uint16_t, uint16_t>(g.s, r, g, map_pitch, unit, taps, stream, timer);
        }
        if (g.bpc == 8) {
            if (fast) return launch_dec_pow2<uint8_t, float>(g.s, r, g, map_pitch, unit, taps, stream, timer);
            return launch_dec_pow2_scalar<uint8_t, float>(g.s, r, g, map_pitch, unit, taps, stream, timer);
        }
        if (fast) return launch_dec_pow2<uint16_t, float>(g.s, r, g, map_pitch, unit, taps, stream, timer);
        return launch_dec_pow2_scalar<uint16_t, float>(g.s, r, g, map_pitch, unit, taps, stream, timer);
    }
    switch (map_kind) {
    case IN_F32: return launch_step<DecNone, float>(r, g, map_pitch, unit, taps, stream, timer);
    case IN_U8: return launch_step<DecNone, uint8_t>(r, g, map_pitch, unit, taps, stream, timer);
    case IN_U16: return launch_step<DecNone, uint16_t>(r, g, map_pitch, unit, taps, stream, timer);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace vqm
