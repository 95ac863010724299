// ss2_pairs.h — exact fp32-pair arithmetic and the ssimulacra2 per-pixel
// terms, shared by the per-scale statistics and the chain's fused column
// pass.
//
// "Research-1363: Device-resident ssimulacra2 and a single-wait MS-SSIM on
// SYCL", Finding 4: the product num_m * num_s of two floats is exact as a
// pair (two_prod); the quotient comes from two correctly rounded fp32
// partial quotients (ff_div, relative error about 2^-46); 1 - q and the edge
// ratio (1 + |r2 - mu2|) / (1 + |r1 - mu1|) - 1 stay pairs; the fourth
// powers are pair products.  Per pixel (fp32, in this order, contraction
// off): num_m = 1 - (mu1 - mu2)^2, num_s = 2 (s12 - mu1 mu2) + C2,
// denom_s = (s11 - mu1^2) + (s22 - mu2^2) + C2, C2 = 0.0009f; then as pairs
// d = max(1 - num_m num_s / denom_s, 0), e as above, art = max(e, 0),
// det = max(-e, 0); the terms d, d^4, art, art^4, det, det^4.
#pragma once

#include <hip/hip_runtime.h>

namespace vqm {
namespace ss2 {

constexpr float kSs2C2 = 0.0009f;

struct Pair {
    float hi, lo;
};

// Knuth's TwoSum: s + e == a + b exactly.
__device__ __forceinline__ Pair two_sum(float a, float b) {
    const float s = a + b;
    const float bb = s - a;
    return Pair{s, (a - (s - bb)) + (b - bb)};
}

// |a| >= |b| or a == 0.
__device__ __forceinline__ Pair fast_two_sum(float a, float b) {
    const float s = a + b;
    return Pair{s, b - (s - a)};
}

// p + e == a b exactly (one fused multiply-add; exact barring underflow).
__device__ __forceinline__ Pair two_prod(float a, float b) {
    const float p = a * b;
    return Pair{p, fmaf(a, b, -p)};
}

__device__ __forceinline__ Pair ff_add(Pair a, Pair b) {
    const Pair s = two_sum(a.hi, b.hi);
    const Pair t = two_sum(a.lo, b.lo);
    const float c = s.lo + t.hi;
    const Pair v = fast_two_sum(s.hi, c);
    const float w = t.lo + v.lo;
    return fast_two_sum(v.hi, w);
}

__device__ __forceinline__ Pair ff_mul(Pair a, Pair b) {
    const Pair p = two_prod(a.hi, b.hi);
    float t = a.hi * b.lo;
    t = fmaf(a.lo, b.hi, t);
    const float e = p.lo + t;
    return fast_two_sum(p.hi, e);
}

// a / b from two correctly rounded fp32 quotients (IEEE division: the
// library is compiled with correctly rounded fp32 divide).
__device__ __forceinline__ Pair ff_div(Pair a, Pair b) {
    const float q1 = a.hi / b.hi;
    const Pair p = two_prod(q1, b.hi);
    float r = (a.hi - p.hi) - p.lo;
    r = r + a.lo;
    r = r - q1 * b.lo;
    const float q2 = r / b.hi;
    return fast_two_sum(q1, q2);
}

__device__ __forceinline__ bool positive(Pair a) { return a.hi > 0.0f || (a.hi == 0.0f && a.lo > 0.0f); }

// The running sum of a thread's terms, all non-negative: the high part is a
// plain fp32 sum, each addition's exact error (TwoSum) goes to the low part,
// and the pair is renormalised every few terms.  Fixed order per thread.
struct Acc {
    float hi = 0.0f, lo = 0.0f;
    __device__ __forceinline__ void add(Pair t) {
        const Pair s = two_sum(hi, t.hi);
        hi = s.hi;
        lo = lo + (s.lo + t.lo);
    }
    __device__ __forceinline__ void norm() {
        const Pair s = fast_two_sum(hi, lo);
        hi = s.hi;
        lo = s.lo;
    }
};

struct Ss2Terms {
    Pair d, d4, art, art4, det, det4;
};

__device__ __forceinline__ Pair fourth_power(Pair a) {
    const Pair a2 = ff_mul(a, a);
    return ff_mul(a2, a2);
}

__device__ __forceinline__ void pixel_terms(float r1, float r2, float m1, float m2, float v11, float v22, float v12,
                                            Acc (&acc)[6]) {
    const float dm = m1 - m2;
    const float num_m = 1.0f - dm * dm;
    const float mu12 = m1 * m2;
    const float num_s = 2.0f * (v12 - mu12) + kSs2C2;
    const float mu11 = m1 * m1, mu22 = m2 * m2;
    const float denom_s = (v11 - mu11) + (v22 - mu22) + kSs2C2;
    // d = 1 - num_m num_s / denom_s as a pair, clamped at 0
    const Pair q = ff_div(two_prod(num_m, num_s), Pair{denom_s, 0.0f});
    Pair d = ff_add(Pair{1.0f, 0.0f}, Pair{-q.hi, -q.lo});
    if (!positive(d)) d = Pair{0.0f, 0.0f};
    acc[0].add(d);
    acc[1].add(fourth_power(d));
    // e = (1 + |r2 - mu2|) / (1 + |r1 - mu1|) - 1; 1 + |x| is exact as a pair
    const float a2 = fabsf(r2 - m2), a1 = fabsf(r1 - m1);
    const Pair ratio = ff_div(two_sum(1.0f, a2), two_sum(1.0f, a1));
    const Pair e = ff_add(ratio, Pair{-1.0f, 0.0f});
    const bool art = positive(e);
    const Pair mag = art ? e : Pair{-e.hi, -e.lo};
    const bool nz = positive(mag);
    const Pair m = nz ? mag : Pair{0.0f, 0.0f};
    const Pair m4 = fourth_power(m);
    const Pair zero{0.0f, 0.0f};
    acc[2].add(art ? m : zero);
    acc[3].add(art ? m4 : zero);
    acc[4].add(art ? zero : m);
    acc[5].add(art ? zero : m4);
}

// Pairs across the 64 lanes of a wave in a fixed butterfly; every lane ends
// with the same bits (ff_add is commutative: each step's parts are exact).
__device__ __forceinline__ Pair wave_pair_sum(Pair v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const Pair o{__shfl_xor(v.hi, off, 64), __shfl_xor(v.lo, off, 64)};
        v = ff_add(v, o);
    }
    return v;
}

// Workgroup sum of six pairs per thread over NT threads: wave butterflies,
// then the waves in index order.  The result is valid in thread 0.
template <int NT>
__device__ __forceinline__ void block_pair_sum(Pair (&v)[6], Pair (*red)[NT / 64]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int k = 0; k < 6; ++k) {
        v[k] = wave_pair_sum(v[k]);
        if (lane == 0) red[k][wave] = v[k];
    }
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int k = 0; k < 6; ++k) {
            Pair t = red[k][0];
            for (int w = 1; w < NT / 64; ++w) t = ff_add(t, red[k][w]);
            v[k] = t;
        }
    }
}

}  // namespace ss2
}  // namespace vqm
