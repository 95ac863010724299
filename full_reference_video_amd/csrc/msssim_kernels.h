// msssim_kernels.h — the MS-SSIM level and finish launchers (library-private).
#pragma once

#include "vqm_kernels.h"

namespace vqm {

// ---------------------------------------------------------------- MS-SSIM

struct MsFrame {
    const void *ref, *dis;       // level planes with row pitch `pitch`
    double *partials;            // this level's 3 spans (l, c, s) of ms_partials(W, H, n) doubles
    float *next_ref, *next_dis;  // floor(W/2) x floor(H/2), pitch next_pitch; NULL at level 5
};
struct MsBatch {
    MsFrame f[kMaxBatch];
};

// Partial sums per span that a batch of n frames writes at a W x H level (the
// grid of the kernel the batch takes), and the most any batch writes.
// `overlapped`: the batch shares the GPU with another batch of its context
// on a second stream, whose work fills the idle SIMDs of its last round of
// strips (the kernel plan then prefers taller strips).
int ms_partials(int W, int H, int n, bool overlapped);
int ms_partials_max(int W, int H);

// One MS-SSIM level of n frames: moments and the l/c/s partial sums of the
// valid region, plus the exact 2x2 mean of the level into the next plane.
hipError_t launch_ms_level(const MsBatch &b, int n, InKind kind, int pitch, int W, int H, int next_pitch,
                           float unit, const Taps &taps, bool overlapped, hipStream_t stream,
                           const KernelTimer &timer);

struct MsFinishFrame {
    const double *partials;      // base of the frame's partials (all levels)
    double *result;              // score (+ 15 means when asked for), device-visible pinned host
};
struct MsFinishBatch {
    MsFinishFrame f[kMaxBatch];
    unsigned lcs_mask;           // bit i: frame i also writes its 15 level means to result[1..15]
};
// Where each level's spans sit in a frame's partials.
struct MsLevels {
    int nb[5];                   // partials per span
    long long offset[5];         // first double of the level's 3 spans
    double count[5];             // valid map pixels of the level
};

// One workgroup per frame: the 15 per-level means from the level spans in a
// fixed tree, and the combined score.
hipError_t launch_ms_finish(const MsFinishBatch &b, int n, const MsLevels &lv, hipStream_t stream);

}  // namespace vqm
