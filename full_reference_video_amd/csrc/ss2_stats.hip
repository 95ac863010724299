// ss2_stats.hip — the ssimulacra2 per-scale statistics on the device, without
// fp64: per pixel and channel the SSIM deficit and the edge ratio as exact
// fp32 pairs, and six sums per channel through a fixed tree.
//
// "Research-1363: Device-resident ssimulacra2 and a single-wait MS-SSIM on
// SYCL", Finding 4: the product num_m * num_s of two floats is exact as a
// pair (two_prod); the quotient comes from two correctly rounded fp32 partial
// quotients (ff_div, relative error about 2^-46); 1 - q and the edge ratio
// (1 + |r2 - mu2|) / (1 + |r1 - mu1|) - 1 stay pairs; the fourth powers are
// pair products; six sums per channel go through a fixed tree (a fixed
// strided pixel subset per work-item, a tree per work-group, one group per
// channel over the partials) whose shape depends only on the plane size, and
// every operation is correctly rounded, so the sums are deterministic.
// Finding 3 gives the reason for pairs: the CPU forms each term in fp64 and
// the fourth powers span too many binades for an exact integer sum.
//
// Per pixel (fp32, in this order, with contraction off):
//   num_m = 1 - (mu1 - mu2)^2, num_s = 2 (s12 - mu1 mu2) + C2,
//   denom_s = (s11 - mu1^2) + (s22 - mu2^2) + C2, C2 = 0.0009f;
// then as pairs: d = max(1 - num_m num_s / denom_s, 0),
//   e = (1 + |r2 - mu2|) / (1 + |r1 - mu1|) - 1, art = max(e, 0),
//   det = max(-e, 0); the sums of d, d^4, art, art^4, det, det^4.
#include "ss2_pairs.h"
#include "ss2_kernels.h"

namespace vqm {
namespace {

using namespace ss2;

constexpr int kNT = 256;
// Seven planes of one channel, in the order of the C ABI.
struct Ss2Channel {
    const float *p[7];  // img1, img2, mu1, mu2, s11, s22, s12
};
struct Ss2Channels {
    Ss2Channel c[kSs2MaxChannels];
};

// Stage 1: workgroup b of channel c.  Thread t of the channel's T = B * kNT
// threads takes the groups of four pixels g = t, t + T, t + 2T, ... (a group
// past the end of the plane is cut short), each group's pixels in order, so
// the order of every addition depends only on the pixel count.  The six
// workgroup sums go to partials[(c * B + b) * 6 + k].
__global__ __launch_bounds__(kNT) void ss2_partials(Ss2Channels ch, long long n, Pair *partials, int vec4) {
    __shared__ Pair red[6][kNT / 64];
    const int c = blockIdx.y, B = gridDim.x;
    const Ss2Channel &pc = ch.c[c];
    const long long groups = (n + 3) / 4;
    const long long T = (long long)B * kNT;
    Acc acc[6];
    int since_norm = 0;
    for (long long g = (long long)blockIdx.x * kNT + threadIdx.x; g < groups; g += T) {
        const long long i0 = 4 * g;
        float v[7][4];
        if (vec4 && i0 + 4 <= n) {
#pragma unroll
            for (int p = 0; p < 7; ++p) {
                const float4 q = *reinterpret_cast<const float4 *>(pc.p[p] + i0);
                v[p][0] = q.x;
                v[p][1] = q.y;
                v[p][2] = q.z;
                v[p][3] = q.w;
            }
        } else {
#pragma unroll
            for (int p = 0; p < 7; ++p)
#pragma unroll
                for (int j = 0; j < 4; ++j) v[p][j] = i0 + j < n ? pc.p[p][i0 + j] : 0.0f;
        }
        const int m = n - i0 < 4 ? (int)(n - i0) : 4;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (j < m) pixel_terms(v[0][j], v[1][j], v[2][j], v[3][j], v[4][j], v[5][j], v[6][j], acc);
        if (++since_norm == 8) {
            since_norm = 0;
#pragma unroll
            for (int k = 0; k < 6; ++k) acc[k].norm();
        }
    }
    Pair s[6];
#pragma unroll
    for (int k = 0; k < 6; ++k) {
        acc[k].norm();
        s[k] = Pair{acc[k].hi, acc[k].lo};
    }
    block_pair_sum<kNT>(s, red);
    if (threadIdx.x == 0) {
#pragma unroll
        for (int k = 0; k < 6; ++k) partials[((long long)c * B + blockIdx.x) * 6 + k] = s[k];
    }
}

// Stage 2: one workgroup per channel sums its B partials of each sum, thread
// t taking partials t, t + kNT, ... in index order, then the workgroup tree.
// The six sums go to result[c * 6 + k] as doubles (hi + lo, one rounding).
__global__ __launch_bounds__(kNT) void ss2_finish(const Pair *partials, int B, double *result) {
    __shared__ Pair red[6][kNT / 64];
    const int c = blockIdx.x;
    Pair s[6];
#pragma unroll
    for (int k = 0; k < 6; ++k) s[k] = Pair{0.0f, 0.0f};
    for (int b = threadIdx.x; b < B; b += kNT)
#pragma unroll
        for (int k = 0; k < 6; ++k) s[k] = ff_add(s[k], partials[((long long)c * B + b) * 6 + k]);
    block_pair_sum<kNT>(s, red);
    if (threadIdx.x == 0) {
#pragma unroll
        for (int k = 0; k < 6; ++k) result[c * 6 + k] = (double)s[k].hi + (double)s[k].lo;
        __threadfence_system();
    }
}

// The pair operations one by one, for the bit-exactness tests: out[i] =
// op(a[i], b[i]) with a pair per element ((hi, lo) interleaved).
__global__ __launch_bounds__(kNT) void pair_ops(int op, const float *a, const float *b, float *out, int n) {
    const int i = blockIdx.x * kNT + threadIdx.x;
    if (i >= n) return;
    const Pair x{a[2 * i], a[2 * i + 1]}, y{b[2 * i], b[2 * i + 1]};
    Pair r{0.0f, 0.0f};
    switch (op) {
    case 0: r = two_sum(x.hi, y.hi); break;
    case 1: r = two_prod(x.hi, y.hi); break;
    case 2: r = ff_add(x, y); break;
    case 3: r = ff_mul(x, y); break;
    case 4: r = ff_div(x, y); break;
    default: break;
    }
    out[2 * i] = r.hi;
    out[2 * i + 1] = r.lo;
}

}  // namespace

int ss2_blocks(long long n) {
    const long long groups = (n + 3) / 4;
    long long b = (groups + (long long)kNT * 8 - 1) / ((long long)kNT * 8);
    if (b < 1) b = 1;
    if (b > kSs2MaxBlocks) b = kSs2MaxBlocks;
    return (int)b;
}

hipError_t launch_ss2_sums(const float *const *planes, int nch, long long n, void *partials, double *result,
                           hipStream_t stream) {
    if (nch < 1 || nch > kSs2MaxChannels || n < 1) return hipErrorInvalidValue;
    Ss2Channels ch;
    int vec4 = 1;
    for (int c = 0; c < nch; ++c)
        for (int p = 0; p < 7; ++p) {
            ch.c[c].p[p] = planes[c * 7 + p];
            if ((uintptr_t)ch.c[c].p[p] & 15u) vec4 = 0;
        }
    const int B = ss2_blocks(n);
    hipLaunchKernelGGL(ss2_partials, dim3(B, nch), dim3(kNT), 0, stream, ch, n, static_cast<Pair *>(partials), vec4);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(ss2_finish, dim3(nch), dim3(kNT), 0, stream, static_cast<const Pair *>(partials), B, result);
    return hipGetLastError();
}

hipError_t launch_pair_ops(int op, const float *a, const float *b, float *out, int n, hipStream_t stream) {
    if (op < 0 || op > 4 || n < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pair_ops, dim3((n + kNT - 1) / kNT), dim3(kNT), 0, stream, op, a, b, out, n);
    return hipGetLastError();
}

}  // namespace vqm
