// ss2_kernels.h — launchers of the ssimulacra2 kernels: the one-scale
// statistics (ss2_stats.hip), the per-scale chain and the downsample
// (ss2_chain.hip).  Kept apart from the float_ssim and MS-SSIM kernels'
// header so that those kernels' sources do not change with these.
#pragma once

#include "vqm_kernels.h"

namespace vqm {

// ---------------------------------------------------------------- ssimulacra2 statistics

constexpr int kSs2MaxChannels = 3;
constexpr int kSs2MaxBlocks = 1024;

// Workgroups per channel of the statistics' first stage for a plane of n
// pixels (a function of n alone, so the tree's shape is too).
int ss2_blocks(long long n);

// The six ssimulacra2 sums of nch channels of n pixels each: planes holds 7
// device pointers per channel (img1, img2, mu1, mu2, s11, s22, s12; fp32,
// tightly packed); partials is device scratch of nch * ss2_blocks(n) * 6
// fp32 pairs; result receives 6 doubles per channel (a device-visible
// address).  Two launches: workgroup partials, then one group per channel.
hipError_t launch_ss2_sums(const float *const *planes, int nch, long long n, void *partials, double *result,
                           hipStream_t stream);

// The pair operations elementwise (0 two_sum, 1 two_prod, 2 ff_add,
// 3 ff_mul, 4 ff_div) over n pairs of device arrays, for the tests.
hipError_t launch_pair_ops(int op, const float *a, const float *b, float *out, int n, hipStream_t stream);

// ---------------------------------------------------------------- ssimulacra2 per-scale chain

constexpr int kSs2MaxScales = 6;

// One scale of the chain: w x h fp32 images a[c], b[c] (tightly packed), the
// row pass's output planes rows[c] (nplanes per channel, pstride floats
// apart), and (optionally, NULL entries for none) the column pass's output
// planes out[c], laid out like rows[c] (may equal rows[c]).
struct Ss2Scale {
    int w, h;
    long long pstride;
    const float *a[kSs2MaxChannels], *b[kSs2MaxChannels];
    float *rows[kSs2MaxChannels];
    float *out[kSs2MaxChannels];
};

// The recursive blur of every scale in two launches (rows, then columns).
// nplanes 5: per channel the five planes a, b, a a, b b, a b; with stats,
// the column pass also forms each workgroup's six ssimulacra2 sums and a
// third launch sums them into result[(s * nch + c) * 6 ..] (6 doubles per
// scale and channel, device-visible).  nplanes 1 (nch 1, no stats): the
// blur of a alone.  coef = {B, a1, a2, a3}.  scratch: device memory of
// ss2_chain_scratch_floats(...) floats (checkpoints and partials).
struct Ss2ChainArgs {
    Ss2Scale scale[kSs2MaxScales];
    int nscales, nch, nplanes;
    bool stats;
    float coef[4];
    float *scratch;
    double *result;
};
size_t ss2_chain_scratch_floats(int nch, int nplanes, const int *w, const int *h, int nscales);
hipError_t launch_ss2_chain(const Ss2ChainArgs &args, hipStream_t stream, const KernelTimer &rows_timer,
                            const KernelTimer &cols_timer);

// ceil(w/2) x ceil(h/2).
void ss2_downsampled_dim(int w, int h, int *ow, int *oh);

// The pyramid of nplanes (up to 6) w x h planes in[i] in one launch:
// out[(l - 1) * nplanes + i] receives the 2x2 downsample of scale l - 1 of
// plane i (scale 0 is in[i]), for l = 1..levels (levels up to 5), each
// tightly packed.
hipError_t launch_ss2_pyramid(const float *const *in, float *const *out, int nplanes, int w, int h, int levels,
                              hipStream_t stream);

}  // namespace vqm
