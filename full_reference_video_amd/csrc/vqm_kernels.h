// vqm_kernels.h — launchers of the gfx950 kernels (library-private).
//
// The runtime (vqm_runtime.cpp) validates every argument, sizes the scratch
// and owns the streams; these launchers only compute grids and enqueue.
//
// Every launcher takes a batch of 1..kMaxBatch frames of the same geometry
// and one launch processes all of them: a lone 2160p frame leaves a couple
// of microseconds of launch ramp-up and drain per kernel that a batch of
// frames shares.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vqm {

constexpr int kMaxBatch = 32;

// The 11 taps of the normalised Gaussian (sigma 1.5) in fp32.
struct Taps {
    float g[11];
};

// Optional kernel timing: when `start` is set, the launch records start and
// stop on the events with the kernel's own begin and end (hipExtLaunchKernel),
// not around the enqueue.
struct KernelTimer {
    hipEvent_t start = nullptr, stop = nullptr;
};

template <typename F, typename... Args>
inline hipError_t launch_kernel(F kernel, dim3 grid, dim3 block, hipStream_t stream, const KernelTimer &t,
                                Args... args) {
    if (t.start != nullptr)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, t.start, t.stop, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
    return hipGetLastError();
}

// Input sample kinds of the SSIM-map and MS-SSIM level kernels.
enum InKind { IN_F32 = 0, IN_U8 = 1, IN_U16 = 2 };

// Offset subtracted from every sample before the moments are formed: the
// middle of the 8-bit scale.  Variances and the covariance do not depend on
// it; it keeps E[x^2] small so fp32 loses less to cancellation.
constexpr float kMomentOffset = 128.0f;

// ---------------------------------------------------------------- float_ssim

struct DecimateFrame {
    const void *ref, *dis;       // raw planes, w x h, tightly packed
    void *out_ref, *out_dis;     // dec_w x dec_h, row pitch dec_pitch samples: fp32 values, or the
                                 // uint16 raw window sums when StepGeometry::packed
};
struct DecimateBatch {
    DecimateFrame f[kMaxBatch];
};

struct SsimFrame {
    const void *ref, *dis;       // map input planes (decimated fp32, or raw at scale 1)
    double *partials;            // >= ssim_partials(dec_w, dec_h) doubles
    double *result;              // device-visible address of the score (and the dB form after it
                                 // when asked for; pinned host memory or device memory)
};
struct SsimBatch {
    SsimFrame f[kMaxBatch];
};

// Geometry shared by every role of a step launch.
struct StepGeometry {
    int w, h, bpc, s;            // raw frame and decimation factor
    float tap;                   // 1.0f / (s * s), formed on the host
    float post;                  // 2^-(2k + bpc - 8) when s = 2^k (power-of-two path)
    int dec_w, dec_h, dec_pitch; // decimated plane (= raw size at scale 1)
    int packed;                  // packed_planes(s, bpc): the decimated planes hold uint16 window sums
};

// Whether the decimated planes can hold the integer sums of the raw window
// samples as uint16 instead of fp32 values: s = 2^k >= 2 with
// bpc + 2k <= 16, so that a window sum (s^2 samples below 2^bpc) fits 16
// bits.  The decimated value is then exactly sum * post (an integer below
// 2^24 times a power of two), so the map reads the same values from half the
// bytes.  2160p 10-bit (s = 8: 10 + 6 = 16), 1080p 8-bit and 853x481 12-bit
// qualify; 16-bit samples at s = 2 do not.
inline bool packed_planes(int s, int bpc) {
    if (s < 2 || (s & (s - 1)) != 0) return false;
    int k = 0;
    while ((1 << k) < s) ++k;
    return bpc + 2 * k <= 16;
}

// The three independent roles of one step launch: decimate one batch, map
// another (whose decimated planes an earlier launch wrote), finish a third
// (whose partials an earlier launch wrote).  Any role may be empty.
struct StepRoles {
    DecimateBatch dec;
    int n_dec;
    int dec_blocks_per_frame;    // filled in by the launcher
    SsimBatch map;
    int n_map;
    SsimBatch fin;               // only partials and result are used
    int n_fin;
    unsigned fin_db_mask;        // bit i: finish frame i also writes its decibel form to result[1]
};

// A step launch passes StepRoles by value with a few small structs beside
// it; the kernel argument block holds at most 4 KiB.
static_assert(sizeof(StepRoles) <= 3584, "step launch arguments exceed the kernel argument block");

// Whether the vectorised power-of-two decimation handles these frames
// (otherwise the general path runs; both compute the same exact sums).
bool decimate_fast_path(const DecimateBatch &b, int n, int w, int h, int bpc, int s);

// Number of partial sums the map role writes per frame.
int ssim_partials(int W, int H);

// One step launch.  map_kind / map_pitch / unit describe the map role's
// input: the decimated planes whenever a decimation role is present (pitch
// dec_pitch; IN_U16 window sums with unit post when g.packed, else IN_F32
// values with unit 1), raw samples (pitch w, unit 2^-(bpc-8)) at scale 1.
hipError_t launch_ssim_step(const StepRoles &r, const StepGeometry &g, InKind map_kind, int map_pitch, float unit,
                            const Taps &taps, hipStream_t stream, const KernelTimer &timer);

// ---------------------------------------------------------------- shared

// XCD-aware block order.  The dispatcher hands consecutive workgroups of a
// grid to the eight XCDs in turn; remapping the linear id so that each XCD
// gets one contiguous range of logical blocks keeps neighbouring tiles (which
// share halo lines) on the same XCD and its L2.
__device__ __forceinline__ void xcd_block(int &bx, int &by, int &bz) {
    const int nx = gridDim.x, ny = gridDim.y;
    const int n = nx * ny * gridDim.z;
    const int L = ((int)blockIdx.z * ny + (int)blockIdx.y) * nx + (int)blockIdx.x;
    const int per = n / 8;
    int Lp = L;
    if (L < per * 8) Lp = (L % 8) * per + L / 8;
    bx = Lp % nx;
    by = (Lp / nx) % ny;
    bz = Lp / (nx * ny);
}

}  // namespace vqm
