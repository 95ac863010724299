// probe.hip — two inspection kernels, not part of the scoring path: a plain
// streaming read of device memory (the HBM read ceiling that the
// decimation's 16-byte non-temporal loads can reach on this GPU), and a
// plain fp32 multiply-add loop (the rate the VALU reaches with ordinary,
// non-packed FMA instructions, against which the arithmetic-bound kernels
// are measured).
#include "probe.h"

namespace vqm {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Workgroup b reads the contiguous chunk of kChunk 16-byte vectors starting
// at b kChunk (the last one is cut short at n): each thread issues its 16
// non-temporal loads (256 apart, so a wave's loads are consecutive) before
// folding them into one word, so the loads are not dead; one word per
// workgroup goes to sink.  Short-lived workgroups, many of them, like the
// decimation's.
constexpr int kLoads = 16;
constexpr long long kChunk = 256LL * kLoads;

__global__ __launch_bounds__(256) void read_probe(const u32x4 *__restrict__ p, long long n, uint32_t *sink) {
    const long long base = (long long)blockIdx.x * kChunk + threadIdx.x;
    u32x4 v[kLoads];
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
        const long long i = base + 256LL * k;
        v[k] = __builtin_nontemporal_load(p + (i < n ? i : n - 1));
    }
    uint32_t acc = 0;
#pragma unroll
    for (int k = 0; k < kLoads; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    __shared__ uint32_t red[256];
    red[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int k = 0; k < 256; ++k) t ^= red[k];
        sink[blockIdx.x] = t;
    }
}

// Each thread runs 16 independent multiply-add chains v = g v + 1 for
// `iters` steps (16 FMAs per step, none waiting on the one before it), then
// stores their sum so that none is dead.  One float per thread to out.
constexpr int kValuChains = 16;

__global__ __launch_bounds__(256) void valu_probe(float *out, int iters, float x) {
    float v[kValuChains];
#pragma unroll
    for (int k = 0; k < kValuChains; ++k) v[k] = x + (float)k + (float)threadIdx.x;
    const float g = x * 0.25f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < kValuChains; ++k) v[k] = __builtin_fmaf(g, v[k], 1.0f);
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < kValuChains; ++k) s += v[k];
    out[(long long)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

long long valu_probe_fmas(int blocks, int iters) { return (long long)blocks * 256 * iters * kValuChains; }

hipError_t launch_valu_probe(float *out, int blocks, int iters, hipStream_t stream, const KernelTimer &timer) {
    if (blocks < 1 || iters < 1) return hipErrorInvalidValue;
    return launch_kernel(valu_probe, dim3((unsigned)blocks), dim3(256), stream, timer, out, iters, 0.5f);
}

long long read_probe_blocks(long long bytes) { return (bytes / 16 + kChunk - 1) / kChunk; }

hipError_t launch_read_probe(const void *buf, long long bytes, uint32_t *sink, hipStream_t stream,
                             const KernelTimer &timer) {
    const long long blocks = read_probe_blocks(bytes);
    if (bytes < 16 || blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    return launch_kernel(read_probe, dim3((unsigned)blocks), dim3(256), stream, timer,
                         static_cast<const u32x4 *>(buf), bytes / 16, sink);
}

}  // namespace vqm
