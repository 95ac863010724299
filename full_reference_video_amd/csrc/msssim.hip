// msssim.hip — one MS-SSIM pyramid level per launch; the last level combines.
//
// "Research-1363: Device-resident ssimulacra2 and a single-wait MS-SSIM on
// SYCL", Finding 6: every scale gets its own span of partial sums, so all
// scales are enqueued at once and the host waits once per frame.  Here the
// spans are summed and combined on the device too (one finish workgroup per
// frame, each span in index order), so one 8-byte score (plus the 15
// per-level means) is the whole read-back.
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

// 32 x 64 tiles, 512 threads: the horizontal pass computes 74 rows for 64
// map rows (16 % halo, against 31 % for 32-row tiles).
constexpr int kTW = 32, kTH = 64, kNT = 512, kRB = 4;
constexpr int kNP = 5;  // moment planes: x, y, x^2, y^2, xy (contrast needs both sigmas)

__constant__ double kBeta[5] = {0.0448, 0.2856, 0.3001, 0.2363, 0.1333};

template <int TW, int TH, int NT, int RB, typename TIn>
__global__ __launch_bounds__(NT) void ms_level(MsBatch b, int pitch, int W, int H, int next_pitch, float unit,
                                               int vec4, Taps taps) {
    constexpr int IH = TH + 10, IP = in_pitch<TW>();
    __shared__ __attribute__((aligned(16))) float lds[tile_lds_floats<TW, TH, kNP>()];
    __shared__ double red[3][NT / 64];
    float *sx = lds, *sy = lds + IH * IP;

    int bx, by, bz;
    xcd_block(bx, by, bz);
    const MsFrame &t = b.f[bz];
    const TIn *ref = static_cast<const TIn *>(t.ref);
    const TIn *dis = static_cast<const TIn *>(t.dis);

    const int MW = W - 10, MH = H - 10;
    const int x0 = bx * TW, y0 = by * TH;

    stage<TW, TH, NT>(ref, dis, pitch, W, H, unit, x0, y0, sx, sy, vec4 != 0);
    __syncthreads();

    // Next level: 2x2 means of this tile's share of the plane, from the
    // staged (offset) samples.  Every step is exact (the sum of four offset
    // samples and the next level's values fit fp32's significand), so adding
    // the offset back gives the same bits as averaging the plain samples.
    // Thread t takes the blocks in columns t % (TW/2) + k TW/2 and rows
    // t / (TW/2) + k NT/(TW/2): one block each in an inner tile (TW/2 x TH/2
    // blocks); the last tile column and row also take the plane's edge.
    if (t.next_ref != nullptr) {
        static_assert(NT % (TW / 2) == 0, "block rows must tile the workgroup");
        constexpr int CW = TW / 2, RS = NT / CW;
        const int xe = (bx == (int)gridDim.x - 1) ? W : x0 + TW;
        const int ye = (by == (int)gridDim.y - 1) ? H : y0 + TH;
        const int nx0 = x0 / 2, ny0 = y0 / 2;
        const int nw = min(xe / 2, W / 2) - nx0, nh = min(ye / 2, H / 2) - ny0;
        for (int r = (int)threadIdx.x / CW; r < nh; r += RS) {
            for (int c = (int)threadIdx.x % CW; c < nw; c += CW) {
                const int l = 2 * r * IP + 2 * c;  // tile-local cell of the block, 8-byte aligned
                const float2 x0v = *reinterpret_cast<const float2 *>(sx + l);
                const float2 x1v = *reinterpret_cast<const float2 *>(sx + l + IP);
                const float2 y0v = *reinterpret_cast<const float2 *>(sy + l);
                const float2 y1v = *reinterpret_cast<const float2 *>(sy + l + IP);
                const int o = (ny0 + r) * next_pitch + nx0 + c;
                t.next_ref[o] = fmaf((x0v.x + x0v.y) + (x1v.x + x1v.y), 0.25f, kMomentOffset);
                t.next_dis[o] = fmaf((y0v.x + y0v.y) + (y1v.x + y1v.y), 0.25f, kMomentOffset);
            }
        }
    }

    horizontal_moments_in_place<TW, TH, NT, kNP>(lds, taps);

    // Per pixel: l = 1 - (mx - my)^2 / (mux^2 + muy^2 + C1) and
    // c = 1 - (sx - sy)^2 / (sx^2 + sy^2 + C2) (the mirrored quotients
    // rewritten, exactly 1 for identical planes), s = (sxy + C3) / (sx sy + C3),
    // with sx^2 = max(var_x, 0).  The three quotients come from one
    // reciprocal of the product of the denominators (at most ~1e14, far
    // inside fp32 range).  For l and c a thread sums only the subtracted
    // parts and takes them from its count of valid pixels at the end.  A
    // thread's few pixels and then its wave are summed in fp32, the waves in
    // fp64.
    constexpr float kC3 = kC2 / 2.0f;
    float dl = 0.0f, dc = 0.0f, ps = 0.0f;
    int npx = 0;
    vertical_moments<TW, TH, NT, RB, kNP>(lds, taps, x0, y0, MW, MH, [&](int, int, const float (&m)[kNP]) {
        const float mx = m[0], my = m[1], xx = m[2], yy = m[3], xy = m[4];
        const float vx = fmaxf(fmaf(-mx, mx, xx), 0.0f);
        const float vy = fmaxf(fmaf(-my, my, yy), 0.0f);
        const float cxy = fmaf(-mx, my, xy);
        const float sdx = hw_sqrt(vx), sdy = hw_sqrt(vy);
        const float ux = mx + kMomentOffset, uy = my + kMomentOffset;
        const float dm = mx - my, ds = sdx - sdy;
        const float d1 = fmaf(ux, ux, fmaf(uy, uy, kC1));
        const float d2 = (vx + vy) + kC2;
        const float d3 = fmaf(sdx, sdy, kC3);
        const float d12 = d1 * d2;
        const float r = rcp(d12 * d3);
        dl = fmaf(dm * dm, (d2 * d3) * r, dl);
        dc = fmaf(ds * ds, (d1 * d3) * r, dc);
        ps = fmaf(cxy + kC3, d12 * r, ps);
        ++npx;
    });
    const float terms[3] = {(float)npx - dl, (float)npx - dc, ps};
    double acc[3];
    block_sum_terms<NT, 3>(terms, red, acc);
    if (threadIdx.x == 0) {
        const int nb = gridDim.x * gridDim.y;
        const int slot = by * gridDim.x + bx;
        t.partials[slot] = acc[0];
        t.partials[nb + slot] = acc[1];
        t.partials[2 * nb + slot] = acc[2];
    }
}

template <int NT>
__global__ __launch_bounds__(NT) void ms_finish(MsFinishBatch b, MsLevels lv) {
    static_assert(NT >= 64, "the powers take one wave");
    __shared__ double red[3][NT / 64];
    __shared__ double lcs[15];
    __shared__ double pw[11];
    const MsFinishFrame &fr = b.f[blockIdx.x];
    for (int j = 0; j < 5; ++j) {
        double tot[3];
        sum_spans<NT, 3>(fr.partials + lv.offset[j], lv.nb[j], (size_t)lv.nb[j], tot, red);
        if (threadIdx.x == 0) {
            lcs[j] = tot[0] / lv.count[j];
            lcs[5 + j] = tot[1] / lv.count[j];
            lcs[10 + j] = tot[2] / lv.count[j];
        }
        __syncthreads();  // red[] is reused by the next level; lcs[] is complete after the last
    }
    // The eleven powers at once, one per lane: L_5^b5, C_j^bj, S_j^bj.
    const int t = threadIdx.x;
    if (t < 11) {
        const int j = t == 0 ? 4 : (t - 1) % 5;
        const double base = t == 0 ? lcs[4] : (t <= 5 ? lcs[5 + j] : lcs[10 + j]);
        pw[t] = pow(base, kBeta[j]);
    }
    __syncthreads();
    if (t != 0) return;
    double ms = pw[0];
    for (int j = 0; j < 5; ++j) {
        const double cj = lcs[5 + j], sj = lcs[10 + j];
        if (!(cj > 0.0) || !(sj > 0.0)) {
            ms = __longlong_as_double(0x7ff8000000000000ll);
            break;
        }
        ms *= pw[1 + j] * pw[6 + j];
    }
    fr.result[0] = ms;
    for (int j = 0; j < 15; ++j) fr.result[1 + j] = lcs[j];
    __threadfence_system();
}

}  // namespace

int ms_partials(int W, int H) {
    return ((W - 10 + kTW - 1) / kTW) * ((H - 10 + kTH - 1) / kTH);
}

hipError_t launch_ms_level(const MsBatch &b, int n, InKind kind, int pitch, int W, int H, int next_pitch,
                           float unit, const Taps &taps, hipStream_t stream, const KernelTimer &timer) {
    if (n < 1 || n > kMaxBatch) return hipErrorInvalidValue;
    const dim3 grid((W - 10 + kTW - 1) / kTW, (H - 10 + kTH - 1) / kTH, n);
    const size_t bytes = kind == IN_F32 ? 4 : (kind == IN_U16 ? 2 : 1);
    int vec4 = 1;
    for (int i = 0; i < n; ++i)
        if (!stage_vec4_ok(b.f[i].ref, pitch, bytes) || !stage_vec4_ok(b.f[i].dis, pitch, bytes)) vec4 = 0;
    switch (kind) {
    case IN_F32:
        return launch_kernel(ms_level<kTW, kTH, kNT, kRB, float>, grid, dim3(kNT), stream, timer, b, pitch, W, H,
                             next_pitch, unit, vec4, taps);
    case IN_U8:
        return launch_kernel(ms_level<kTW, kTH, kNT, kRB, uint8_t>, grid, dim3(kNT), stream, timer, b, pitch, W, H,
                             next_pitch, unit, vec4, taps);
    case IN_U16:
        return launch_kernel(ms_level<kTW, kTH, kNT, kRB, uint16_t>, grid, dim3(kNT), stream, timer, b, pitch, W,
                             H, next_pitch, unit, vec4, taps);
    default:
        return hipErrorInvalidValue;
    }
}

hipError_t launch_ms_finish(const MsFinishBatch &b, int n, const MsLevels &lv, hipStream_t stream) {
    if (n < 1 || n > kMaxBatch) return hipErrorInvalidValue;
    hipLaunchKernelGGL(ms_finish<256>, dim3(n), dim3(256), 0, stream, b, lv);
    return hipGetLastError();
}

}  // namespace vqm
