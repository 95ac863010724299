// ssim.hip — fused 11x11 Gaussian moments, SSIM map and fixed-tree mean.
//
// "ADR-1405: float_ssim_hip decimates on the device, bit-identical to the
// CPU", Context and Decision 3–4: on the decimated planes (or on the raw
// samples directly at scale 1) the 11x11 Gaussian local means, variances and
// covariance give a per-pixel SSIM term over the valid region, whose mean is
// the frame score; one read-back per frame.
// "Research-1363: Device-resident ssimulacra2 and a single-wait MS-SSIM on
// SYCL", Finding 4: the sum runs through a fixed tree — a fixed pixel subset
// per work-item, a tree per work-group, one group over the partials — so the
// result depends only on the plane size.
//
// One workgroup per TW x TH tile of the map.  The tile's (TW+10) x (TH+10)
// input window of both planes is staged in LDS, the horizontal 11-tap pass
// writes five moment planes to LDS (four columns per thread step), and the
// vertical pass (four rows per thread step) forms the moments of each map
// pixel and its SSIM term in fp32, with the mid-scale offset removed first
// so E[x^2] - mu^2 cancels less.  Each thread adds its map
// pixels in fp64; the workgroup sum goes to a partials array, and a finish
// kernel (one workgroup per frame) sums the partials in index order and
// writes the mean straight into the pinned host result slot.
#include "ssim_common.h"

namespace vqm {
namespace {

constexpr int kTW = 32, kTH = 32, kNT = 256, kRB = 4;

template <int TW, int TH, int NT, int RB, typename TIn>
__global__ __launch_bounds__(NT) void ssim_map(SsimBatch b, int pitch, int W, int H, float unit, Taps taps) {
    constexpr int IH = TH + 10, IP = in_pitch<TW>();
    __shared__ __attribute__((aligned(16))) float sx[IH * IP];
    __shared__ __attribute__((aligned(16))) float sy[IH * IP];
    __shared__ __attribute__((aligned(16))) float hm[5 * IH * TW];
    __shared__ double red[1][NT / 64];

    int bx, by, bz;
    xcd_block(bx, by, bz);
    const SsimFrame &fr = b.f[bz];
    const TIn *ref = static_cast<const TIn *>(fr.ref);
    const TIn *dis = static_cast<const TIn *>(fr.dis);

    const int MW = W - 10, MH = H - 10;
    const int x0 = bx * TW, y0 = by * TH;

    stage<TW, TH, NT>(ref, dis, pitch, W, H, unit, x0, y0, sx, sy);
    __syncthreads();
    horizontal_moments<TW, TH, NT>(sx, sy, taps, hm);
    __syncthreads();

    double acc[1] = {0.0};
    vertical_moments<TW, TH, NT, RB>(hm, taps, x0, y0, MW, MH,
                                     [&](int, int, float mx, float my, float xx, float yy, float xy) {
        const float sxx = xx - mx * mx;
        const float syy = yy - my * my;
        const float sxy = xy - mx * my;
        const float ux = mx + kMomentOffset;
        const float uy = my + kMomentOffset;
        // Numerator and denominator as mirror images (contraction is off),
        // so identical planes give exactly 1.
        const float num = (ux * uy + ux * uy + kC1) * (sxy + sxy + kC2);
        const float den = (ux * ux + uy * uy + kC1) * (sxx + syy + kC2);
        acc[0] += (double)(num / den);
    });

    block_sum<NT, 1>(acc, red);
    if (threadIdx.x == 0) fr.partials[by * gridDim.x + bx] = acc[0];
}

// One workgroup per frame: the fixed-tree sum of the frame's partials, the
// mean, and its 8-byte write to the pinned host result slot.
template <int NT>
__global__ __launch_bounds__(NT) void ssim_finish(SsimBatch b, int nb, double count) {
    __shared__ double red[1][NT / 64];
    const SsimFrame &fr = b.f[blockIdx.x];
    double tot[1];
    sum_spans<NT, 1>(fr.partials, nb, 0, tot, red);
    if (threadIdx.x == 0) {
        *fr.result = tot[0] / count;
        __threadfence_system();
    }
}

}  // namespace

int ssim_partials(int W, int H) {
    return ((W - 10 + kTW - 1) / kTW) * ((H - 10 + kTH - 1) / kTH);
}

hipError_t launch_ssim(const SsimBatch &b, int n, InKind kind, int pitch, int W, int H, float unit,
                       const Taps &taps, hipStream_t stream) {
    if (n < 1 || n > kMaxBatch) return hipErrorInvalidValue;
    const dim3 grid((W - 10 + kTW - 1) / kTW, (H - 10 + kTH - 1) / kTH, n);
    switch (kind) {
    case IN_F32:
        hipLaunchKernelGGL((ssim_map<kTW, kTH, kNT, kRB, float>), grid, dim3(kNT), 0, stream, b, pitch, W, H, unit, taps);
        break;
    case IN_U8:
        hipLaunchKernelGGL((ssim_map<kTW, kTH, kNT, kRB, uint8_t>), grid, dim3(kNT), 0, stream, b, pitch, W, H, unit, taps);
        break;
    case IN_U16:
        hipLaunchKernelGGL((ssim_map<kTW, kTH, kNT, kRB, uint16_t>), grid, dim3(kNT), 0, stream, b, pitch, W, H, unit,
                           taps);
        break;
    default:
        return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const double count = (double)(W - 10) * (double)(H - 10);
    hipLaunchKernelGGL(ssim_finish<256>, dim3(n), dim3(256), 0, stream, b, (int)(grid.x * grid.y), count);
    return hipGetLastError();
}

}  // namespace vqm
