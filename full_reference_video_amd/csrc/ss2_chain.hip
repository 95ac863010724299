// ss2_chain.hip — the ssimulacra2 per-scale chain on the device: the three
// multiplies, the recursive blur along every row and then every column, and
// the 2x2 downsample to the next scale.  The six sums per channel come from
// ss2_stats.hip.
//
// "Research-1363: Device-resident ssimulacra2 and a single-wait MS-SSIM on
// SYCL", Finding 2: with contraction off and every product its own rounded
// value, the multiplies, both blur passes and the downsample reproduce the
// CPU bit for bit; Finding 7: the blur is a sequential recurrence along each
// line, so a pass has one work-item per row or column, five blurs per
// channel and scale.  The recursion (third order, caller coefficients
// B, a1, a2, a3, at rest outside the line), causal then anticausal:
//   w[i] = ((B x[i] + a3 w[i-3]) + a2 w[i-2]) + a1 w[i-1]
//   y[i] = ((B w[i] + a3 y[i+3]) + a2 y[i+2]) + a1 y[i+1]
// (the library is compiled with -ffp-contract=off, so each product here is
// rounded on its own).
//
// Row pass.  The page's horizontal walk makes every lane of a load touch its
// own cache line.  Here a workgroup owns 64 rows of one channel, one wave
// per blurred plane (lane = row); 32-column chunks of the two images are
// loaded row-contiguously into LDS, each lane walks its row through the
// chunk (forming its plane's product on the fly, so the multiplies cost no
// pass of their own), and the chunk's outputs leave LDS row-contiguously
// again.  The causal outputs go to the output planes, and the anticausal
// walk reads them back chunk by chunk from the right and overwrites them.
// Column pass: lanes own consecutive columns (loads already contiguous
// across the wave); it runs in place on the row pass's output.
#include "vqm_kernels.h"

#include <algorithm>

namespace vqm {
namespace {

constexpr int kRowsPerGroup = 64;  // one row per lane
constexpr int kChunk = 32;         // columns per LDS chunk
constexpr int kPitch = kChunk + 1; // odd pitch: a lane per row reads distinct banks
constexpr int kColBatch = 8;       // rows loaded together by a column walk

struct Coef {
    float B, a1, a2, a3;
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

struct RowPass {
    const float *a[kSs2MaxChannels], *b[kSs2MaxChannels];
    float *out[kSs2MaxChannels];  // NP planes per channel, pstride floats apart
};

// The blurred plane p of a lane, from the two images' samples: a, b, a a,
// b b, a b (p is uniform across a wave).
template <int NP>
__device__ __forceinline__ float plane_input(int p, float xa, float xb) {
    if (NP == 1) return xa;
    const float aa = xa * xa, bb = xb * xb, ab = xa * xb;
    return p == 0 ? xa : p == 1 ? xb : p == 2 ? aa : p == 3 ? bb : ab;
}

template <int NP>
__global__ __launch_bounds__(64 * NP) void ss2_rows(RowPass rp, int w, int h, long long pstride, Coef k) {
    constexpr int NT = 64 * NP;
    constexpr int NI = NP == 1 ? 1 : 2;  // image tiles
    __shared__ float tin[NI][kRowsPerGroup][kPitch];
    __shared__ float tout[NP][kRowsPerGroup][kPitch];

    const int c = blockIdx.y;
    const int r0 = blockIdx.x * kRowsPerGroup;
    const int nrows = min(kRowsPerGroup, h - r0);
    const int p = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const float *img[2] = {rp.a[c], NP == 1 ? rp.a[c] : rp.b[c]};
    float *const out = rp.out[c] + (long long)p * pstride;
    const int nchunks = (w + kChunk - 1) / kChunk;
    // a thread's share of a tile: column t % kChunk, rows t / kChunk + i NT / kChunk
    const int tcol = threadIdx.x % kChunk, trow = threadIdx.x / kChunk;
    // a wave's share of its own plane's tile: column lane % kChunk, rows lane / kChunk + 2i
    const int wcol = lane % kChunk, wrow = lane / kChunk;

    // causal walk, left to right
    float s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
    for (int ch = 0; ch < nchunks; ++ch) {
        const int c0 = ch * kChunk, n = min(kChunk, w - c0);
        if (tcol < n) {
#pragma unroll
            for (int t = 0; t < NI; ++t)
                for (int i = trow; i < nrows; i += NT / kChunk)
                    tin[t][i][tcol] = img[t][(long long)(r0 + i) * w + c0 + tcol];
        }
        __syncthreads();
        if (lane < nrows) {
            for (int j = 0; j < n; ++j) {
                const float x = plane_input<NP>(p, tin[0][lane][j], tin[NI - 1][lane][j]);
                const float v = recur(k, x, s1, s2, s3);
                tout[p][lane][j] = v;
                s3 = s2;
                s2 = s1;
                s1 = v;
            }
        }
        __syncthreads();
        if (wcol < n)
            for (int i = wrow; i < nrows; i += 2) out[(long long)(r0 + i) * w + c0 + wcol] = tout[p][i][wcol];
        // the next chunk's first barrier orders these reads of tout before
        // its walk writes tout again
    }

    // anticausal walk, right to left, over the causal outputs (each wave
    // reads and writes only its own plane's tile)
    float q1 = 0.0f, q2 = 0.0f, q3 = 0.0f;
    for (int ch = nchunks - 1; ch >= 0; --ch) {
        const int c0 = ch * kChunk, n = min(kChunk, w - c0);
        __syncthreads();
        if (wcol < n)
            for (int i = wrow; i < nrows; i += 2) tout[p][i][wcol] = out[(long long)(r0 + i) * w + c0 + wcol];
        __syncthreads();
        if (lane < nrows) {
            for (int j = n - 1; j >= 0; --j) {
                const float v = recur(k, tout[p][lane][j], q1, q2, q3);
                tout[p][lane][j] = v;
                q3 = q2;
                q2 = q1;
                q1 = v;
            }
        }
        __syncthreads();
        if (wcol < n)
            for (int i = wrow; i < nrows; i += 2) out[(long long)(r0 + i) * w + c0 + wcol] = tout[p][i][wcol];
    }
}

struct ColPass {
    float *planes[kSs2MaxChannels];  // NP planes per channel, pstride floats apart
};

// In place: each lane walks one column of one plane, kColBatch rows loaded
// before any of them is used.
template <int NP>
__global__ __launch_bounds__(64 * NP) void ss2_cols(ColPass cp, int w, int h, long long pstride, Coef k) {
    const int c = blockIdx.y;
    const int p = threadIdx.x >> 6;
    const int x = blockIdx.x * 64 + (threadIdx.x & 63);
    if (x >= w) return;  // no barriers below
    float *const col = cp.planes[c] + (long long)p * pstride + x;
    const long long W = w;

    float s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
    int r = 0;
    for (; r + kColBatch <= h; r += kColBatch) {
        float v[kColBatch];
#pragma unroll
        for (int i = 0; i < kColBatch; ++i) v[i] = col[(r + i) * W];
#pragma unroll
        for (int i = 0; i < kColBatch; ++i) {
            const float y = recur(k, v[i], s1, s2, s3);
            s3 = s2;
            s2 = s1;
            s1 = y;
            v[i] = y;
        }
#pragma unroll
        for (int i = 0; i < kColBatch; ++i) col[(r + i) * W] = v[i];
    }
    for (; r < h; ++r) {
        const float y = recur(k, col[r * W], s1, s2, s3);
        s3 = s2;
        s2 = s1;
        s1 = y;
        col[r * W] = y;
    }

    s1 = s2 = s3 = 0.0f;
    r = h;
    for (; r - kColBatch >= 0; r -= kColBatch) {
        float v[kColBatch];  // v[i] is row r - 1 - i
#pragma unroll
        for (int i = 0; i < kColBatch; ++i) v[i] = col[(r - 1 - i) * W];
#pragma unroll
        for (int i = 0; i < kColBatch; ++i) {
            const float y = recur(k, v[i], s1, s2, s3);
            s3 = s2;
            s2 = s1;
            s1 = y;
            v[i] = y;
        }
#pragma unroll
        for (int i = 0; i < kColBatch; ++i) col[(r - 1 - i) * W] = v[i];
    }
    for (; r > 0; --r) {
        const float y = recur(k, col[(r - 1) * W], s1, s2, s3);
        s3 = s2;
        s2 = s1;
        s1 = y;
        col[(r - 1) * W] = y;
    }
}

struct DownPass {
    const float *in[2 * kSs2MaxChannels];
    float *out[2 * kSs2MaxChannels];
};

// ceil(w/2) x ceil(h/2) means of 2x2 blocks, the last column and row
// repeated when the size is odd: ((a + b) + (c + d)) * 0.25f, a and b from
// the upper row.
__global__ __launch_bounds__(256) void ss2_down(DownPass d, int w, int h, int ow, int oh) {
    const float *in = d.in[blockIdx.y];
    float *out = d.out[blockIdx.y];
    const long long n = (long long)ow * oh;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
        const int y = (int)(i / ow), x = (int)(i % ow);
        const int r0 = 2 * y, r1 = min(2 * y + 1, h - 1);
        const int c0 = 2 * x, c1 = min(2 * x + 1, w - 1);
        const float a = in[(long long)r0 * w + c0], b = in[(long long)r0 * w + c1];
        const float cc = in[(long long)r1 * w + c0], dd = in[(long long)r1 * w + c1];
        out[i] = ((a + b) + (cc + dd)) * 0.25f;
    }
}

Coef coef_of(const float coef[4]) { return Coef{coef[0], coef[1], coef[2], coef[3]}; }

}  // namespace

hipError_t launch_ss2_rows(const float *const *a, const float *const *b, float *const *out, int nch, int nplanes,
                           int w, int h, long long pstride, const float coef[4], hipStream_t stream,
                           const KernelTimer &timer) {
    if (nch < 1 || nch > kSs2MaxChannels || w < 1 || h < 1 || (nplanes != 1 && nplanes != 5))
        return hipErrorInvalidValue;
    RowPass rp{};
    for (int c = 0; c < nch; ++c) {
        rp.a[c] = a[c];
        rp.b[c] = nplanes == 5 ? b[c] : a[c];
        rp.out[c] = out[c];
    }
    const dim3 grid((h + kRowsPerGroup - 1) / kRowsPerGroup, nch);
    if (nplanes == 5)
        return launch_kernel(ss2_rows<5>, grid, dim3(320), stream, timer, rp, w, h, pstride, coef_of(coef));
    return launch_kernel(ss2_rows<1>, grid, dim3(64), stream, timer, rp, w, h, pstride, coef_of(coef));
}

hipError_t launch_ss2_cols(float *const *planes, int nch, int nplanes, int w, int h, long long pstride,
                           const float coef[4], hipStream_t stream, const KernelTimer &timer) {
    if (nch < 1 || nch > kSs2MaxChannels || w < 1 || h < 1 || (nplanes != 1 && nplanes != 5))
        return hipErrorInvalidValue;
    ColPass cp{};
    for (int c = 0; c < nch; ++c) cp.planes[c] = planes[c];
    const dim3 grid((w + 63) / 64, nch);
    if (nplanes == 5)
        return launch_kernel(ss2_cols<5>, grid, dim3(320), stream, timer, cp, w, h, pstride, coef_of(coef));
    return launch_kernel(ss2_cols<1>, grid, dim3(64), stream, timer, cp, w, h, pstride, coef_of(coef));
}

void ss2_downsampled_dim(int w, int h, int *ow, int *oh) {
    *ow = (w + 1) / 2;
    *oh = (h + 1) / 2;
}

hipError_t launch_ss2_down(const float *const *in, float *const *out, int nplanes, int w, int h,
                           hipStream_t stream) {
    if (nplanes < 1 || nplanes > 2 * kSs2MaxChannels || w < 1 || h < 1) return hipErrorInvalidValue;
    DownPass d{};
    for (int i = 0; i < nplanes; ++i) {
        d.in[i] = in[i];
        d.out[i] = out[i];
    }
    int ow, oh;
    ss2_downsampled_dim(w, h, &ow, &oh);
    const long long n = (long long)ow * oh;
    const long long blocks = std::min<long long>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(ss2_down, dim3((unsigned)blocks, nplanes), dim3(256), 0, stream, d, w, h, ow, oh);
    return hipGetLastError();
}

}  // namespace vqm
