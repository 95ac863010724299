// vqm_kernels.h — launchers of the gfx950 kernels (library-private).
//
// The runtime (vqm_runtime.cpp) validates every argument, sizes the scratch
// and owns the streams; these launchers only compute grids and enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vqm {

// The 11 taps of the normalised Gaussian (sigma 1.5) in fp32.
struct Taps {
    float g[11];
};

// Input sample kinds of the SSIM-map and MS-SSIM level kernels.
enum InKind { IN_F32 = 0, IN_U8 = 1, IN_U16 = 2 };

// Offset subtracted from every sample before the moments are formed: the
// middle of the 8-bit scale.  Variances and the covariance do not depend on
// it; it keeps E[x^2] small so fp32 loses less to cancellation.
constexpr float kMomentOffset = 128.0f;

// ---------------------------------------------------------------- decimation

// Whether the vectorised power-of-two decimation kernel handles this frame
// (otherwise the general kernel runs; both are exact).
bool decimate_fast_path(const void *ref, const void *dis, int w, int h, int bpc, int s);

// Box low-pass and decimate both planes: out_* are dec_w x dec_h floats with
// a row pitch of `opitch` floats.  `tap` = 1.0f/(s*s) formed by the caller.
hipError_t launch_decimate(const void *ref, const void *dis, int w, int h, int bpc, int s,
                           float tap, float *out_ref, float *out_dis, int dec_w, int dec_h,
                           int opitch, hipStream_t stream);

// ---------------------------------------------------------------- SSIM map

// Device-side state of one reduction: one partial per workgroup, a ticket
// counter that is zero at rest, and where the final value goes.
struct ReduceTarget {
    double *partials;     // >= ssim_partials(...) doubles
    unsigned *ticket;     // one counter, zero between launches
    double *result;       // device-visible pointer to the score (pinned host)
};

// Number of partial sums the SSIM-map kernel writes for a W x H plane.
int ssim_partials(int W, int H);

// Fused 11x11 Gaussian moments + SSIM map + fixed-tree mean over the valid
// (W-10) x (H-10) region of two planes with row pitch `pitch` samples.
// Raw planes (IN_U8 / IN_U16) are scaled by `unit` = 2^-(bpc-8).
hipError_t launch_ssim(const void *ref, const void *dis, InKind kind, int pitch, int W, int H,
                       float unit, const Taps &taps, ReduceTarget rt, hipStream_t stream);

// ---------------------------------------------------------------- MS-SSIM

struct MsLevelTarget {
    double *partials;     // 3 * ms_partials(W, H) doubles (l, c, s spans)
    unsigned *ticket;     // one counter per level, zero at rest
    double *lcs_dev;      // 15 doubles: L1..L5, C1..C5, S1..S5 (device)
    double *result;       // score + 15 means, device-visible pinned host (last level)
    float *next_ref;      // floor(W/2) x floor(H/2) plane, pitch next_pitch; NULL at level 5
    float *next_dis;
    int next_pitch;
};

int ms_partials(int W, int H);

// One MS-SSIM level `level` (0..4): moments and l/c/s means of the valid
// region, plus the exact 2x2 mean of the level into the next plane.  The
// last level also combines the 15 means into the score.
hipError_t launch_ms_level(const void *ref, const void *dis, InKind kind, int pitch, int W, int H,
                           float unit, const Taps &taps, int level, MsLevelTarget t,
                           hipStream_t stream);

}  // namespace vqm
