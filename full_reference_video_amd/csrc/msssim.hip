// msssim.hip — one MS-SSIM pyramid level per launch; the last level combines.
//
// "Research-1363: Device-resident ssimulacra2 and a single-wait MS-SSIM on
// SYCL", Finding 6: every scale gets its own span of partial sums, so all
// scales are enqueued at once and the host waits once per frame.  Here the
// combine runs on the device too, so one 8-byte score (plus the 15 per-level
// means) is the whole read-back.
//
// Level j of the pyramid is the full-resolution sample plane for j = 1 and the
// exact 2x2 mean ((a + b) + (c + d)) * 0.25f of level j-1 after that.  Per
// level, on the valid (W-10) x (H-10) region: luminance
// (2 mx my + C1)/(mx^2 + my^2 + C1), contrast (2 sx sy + C2)/(sx^2 + sy^2 + C2)
// and structure (sxy + C3)/(sx sy + C3), C3 = C2/2, sx = sqrt(max(var, 0));
// their means L_j, C_j, S_j.  The score is
// L_5^b5 * prod_j C_j^b_j * S_j^b_j, b = {0.0448, 0.2856, 0.3001, 0.2363,
// 0.1333} (the published MS-SSIM weights), NaN when any C_j or S_j <= 0.
//
// The tile kernel is the SSIM-map kernel's (LDS-staged halo tile, separable
// 11-tap moments) with three fp64 sums per thread, plus the downsample: each
// workgroup writes the next level's pixels whose 2x2 block starts inside its
// own tile (the last tile column/row also takes the plane's remaining edge),
// so every pixel of the next level is written exactly once.
#include "ssim_common.h"

namespace vqm {
namespace {

constexpr int kTW = 64, kTH = 16, kNT = 256;

__constant__ double kBeta[5] = {0.0448, 0.2856, 0.3001, 0.2363, 0.1333};

template <int TW, int TH, int NT, typename TIn>
__global__ __launch_bounds__(NT) void ms_level(const TIn *__restrict__ ref, const TIn *__restrict__ dis,
                                               int pitch, int W, int H, float unit, Taps taps, int level,
                                               MsLevelTarget t) {
    constexpr int IW = TW + 10, IH = TH + 10;
    __shared__ float sx[IH * IW], sy[IH * IW];
    __shared__ float hmx[IH * TW], hmy[IH * TW], hxx[IH * TW], hyy[IH * TW], hxy[IH * TW];
    __shared__ double red[3][NT / 64];
    __shared__ int is_last;

    const int MW = W - 10, MH = H - 10;
    const int x0 = blockIdx.x * TW, y0 = blockIdx.y * TH;

    stage_tile<TW, TH, NT>(ref, dis, pitch, W, H, unit, x0, y0, sx, sy);
    __syncthreads();

    // Next level: 2x2 means of this tile's share of the plane, from the
    // staged (offset) samples.  Every step is exact, so adding the offset
    // back gives the same bits as averaging the plain samples.
    if (t.next_ref != nullptr) {
        const int xe = (blockIdx.x == gridDim.x - 1) ? W : x0 + TW;
        const int ye = (blockIdx.y == gridDim.y - 1) ? H : y0 + TH;
        const int nx0 = x0 / 2, ny0 = y0 / 2;
        const int nxe = min(xe / 2, W / 2), nye = min(ye / 2, H / 2);
        const int nw = nxe - nx0, nh = nye - ny0;
        for (int i = threadIdx.x; i < nw * nh; i += NT) {
            const int r = i / nw, c = i - r * nw;
            const int lr = 2 * r, lc = 2 * c;  // tile-local position of the block
            const float a = sx[lr * IW + lc], b = sx[lr * IW + lc + 1];
            const float cc = sx[(lr + 1) * IW + lc], d = sx[(lr + 1) * IW + lc + 1];
            const float e = sy[lr * IW + lc], f = sy[lr * IW + lc + 1];
            const float g = sy[(lr + 1) * IW + lc], hh = sy[(lr + 1) * IW + lc + 1];
            const size_t o = (size_t)(ny0 + r) * (size_t)t.next_pitch + (size_t)(nx0 + c);
            t.next_ref[o] = ((a + b) + (cc + d)) * 0.25f + kMomentOffset;
            t.next_dis[o] = ((e + f) + (g + hh)) * 0.25f + kMomentOffset;
        }
    }

    horizontal_moments<TW, TH, NT>(sx, sy, taps, hmx, hmy, hxx, hyy, hxy);
    __syncthreads();

    constexpr float kC3 = kC2 / 2.0f;
    double acc[3] = {0.0, 0.0, 0.0};
    for (int i = threadIdx.x; i < TH * TW; i += NT) {
        const int r = i / TW, c = i - r * TW;
        if (x0 + c < MW && y0 + r < MH) {
            float mx, my, xx, yy, xy;
            vertical_moments<TW>(hmx, hmy, hxx, hyy, hxy, taps, r, c, mx, my, xx, yy, xy);
            const float vx = xx - mx * mx;
            const float vy = yy - my * my;
            const float cxy = xy - mx * my;
            const float sdx = sqrtf(fmaxf(vx, 0.0f));
            const float sdy = sqrtf(fmaxf(vy, 0.0f));
            const float ux = mx + kMomentOffset;
            const float uy = my + kMomentOffset;
            const float l = (ux * uy + ux * uy + kC1) / (ux * ux + uy * uy + kC1);
            const float cs = (sdx * sdy + sdx * sdy + kC2) / (sdx * sdx + sdy * sdy + kC2);
            const float st = (cxy + kC3) / (sdx * sdy + kC3);
            acc[0] += (double)l;
            acc[1] += (double)cs;
            acc[2] += (double)st;
        }
    }

    block_sum<NT, 3>(acc, red);
    const int nb = gridDim.x * gridDim.y;
    const int slot = blockIdx.y * gridDim.x + blockIdx.x;
    if (!publish_and_elect<NT, 3>(acc, t.partials, nb, slot, t.ticket, &is_last)) return;

    double tot[3];
    finish_spans<NT, 3>(t.partials, nb, t.ticket, tot, red);
    if (threadIdx.x == 0) {
        const double n = (double)MW * (double)MH;
        const double L = tot[0] / n, C = tot[1] / n, S = tot[2] / n;
        t.lcs_dev[level] = L;
        t.lcs_dev[5 + level] = C;
        t.lcs_dev[10 + level] = S;
        if (level == 4) {
            // Earlier levels' means were written by earlier launches on the
            // same stream.
            double lcs[15];
            for (int j = 0; j < 15; ++j) lcs[j] = load_agent(t.lcs_dev + j);
            lcs[4] = L;
            lcs[9] = C;
            lcs[14] = S;
            double ms = pow(lcs[4], kBeta[4]);
            for (int j = 0; j < 5; ++j) {
                const double cj = lcs[5 + j], sj = lcs[10 + j];
                if (!(cj > 0.0) || !(sj > 0.0)) {
                    ms = __longlong_as_double(0x7ff8000000000000ll);
                    break;
                }
                ms *= pow(cj, kBeta[j]) * pow(sj, kBeta[j]);
            }
            t.result[0] = ms;
            for (int j = 0; j < 15; ++j) t.result[1 + j] = lcs[j];
            __threadfence_system();
        }
    }
}

}  // namespace

int ms_partials(int W, int H) {
    return ((W - 10 + kTW - 1) / kTW) * ((H - 10 + kTH - 1) / kTH);
}

hipError_t launch_ms_level(const void *ref, const void *dis, InKind kind, int pitch, int W, int H,
                           float unit, const Taps &taps, int level, MsLevelTarget t,
                           hipStream_t stream) {
    const dim3 grid((W - 10 + kTW - 1) / kTW, (H - 10 + kTH - 1) / kTH);
    switch (kind) {
    case IN_F32:
        hipLaunchKernelGGL((ms_level<kTW, kTH, kNT, float>), grid, dim3(kNT), 0, stream,
                           static_cast<const float *>(ref), static_cast<const float *>(dis), pitch, W,
                           H, unit, taps, level, t);
        break;
    case IN_U8:
        hipLaunchKernelGGL((ms_level<kTW, kTH, kNT, uint8_t>), grid, dim3(kNT), 0, stream,
                           static_cast<const uint8_t *>(ref), static_cast<const uint8_t *>(dis), pitch,
                           W, H, unit, taps, level, t);
        break;
    case IN_U16:
        hipLaunchKernelGGL((ms_level<kTW, kTH, kNT, uint16_t>), grid, dim3(kNT), 0, stream,
                           static_cast<const uint16_t *>(ref), static_cast<const uint16_t *>(dis),
                           pitch, W, H, unit, taps, level, t);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace vqm
