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
// Two level kernels compute the same per-pixel moments and terms, bit for
// bit (the same products and 11-tap sums in the same order, and one shared
// term function), and each writes every pixel of the next level exactly once:
// - the tile kernel is the SSIM-map kernel's (LDS-staged halo tile,
//   separable 11-tap moments) plus the downsample of the 2x2 blocks that
//   start inside its tile (the last tile column/row also takes the plane's
//   remaining edge);
// - the row-streaming kernel walks 128-column strips down the plane with the
//   vertical filter in registers (below).
// The per-pixel terms are summed exactly as integers, so which kernel ran,
// and how it split the plane, does not change a single bit of the score; the
// launcher picks per level and batch size (ms_plan).  Both ideas have a
// precedent in "ADR-1357: Run the SYCL CAMBI extractor entirely on the
// device", Decision: there a work-item owns a column and slides its window
// down the rows, and the pooled sum is formed exactly as an integer in units
// of 2^-24.
#include "msssim_kernels.h"
#include "ssim_common.h"

#include <algorithm>
#include <utility>

namespace vqm {
namespace {

// 32 x 64 tiles, 512 threads: the horizontal pass computes 74 rows for 64
// map rows (16 % halo, against 31 % for 32-row tiles).
constexpr int kTW = 32, kTH = 64, kNT = 512, kRB = 4;
constexpr int kNP = 5;  // moment planes: x, y, x^2, y^2, xy (contrast needs both sigmas)

__constant__ double kBeta[5] = {0.0448, 0.2856, 0.3001, 0.2363, 0.1333};

// One map pixel's terms from its five moments (means with the offset
// removed, raw second moments): the luminance and contrast deficits 1 - l and
// 1 - c and the structure s, each in units of 2^-24 truncated toward zero.
// l = 1 - (mx - my)^2 / (mux^2 + muy^2 + C1) and
// c = 1 - (sx - sy)^2 / (sx^2 + sy^2 + C2) (the mirrored quotients
// rewritten, so identical planes give deficits of exactly 0),
// s = (sxy + C3) / (sx sy + C3), with sx^2 = |var_x| (a variance whose fp32
// value comes out below zero is a rounding error of a few ulps of the second
// moment, far below C2; its magnitude costs nothing: the consumers take it as
// an input modifier); the three quotients share one reciprocal of the product
// of the denominators (at most ~1e14).  Both level kernels take every pixel
// through this function and add the integers exactly (a level's sums stay far
// below 2^53 in fp64), so the sums, and the score, do not depend on which
// kernel ran, how it split the plane, or how many frames shared the launch.
// Truncation moves a mean by less than 2^-24.
struct LcsAcc {
    int dl = 0, dc = 0, s = 0;
};

__device__ __forceinline__ void ms_pixel(const float (&m)[5], LcsAcc &a) {
    constexpr float kC3 = kC2 / 2.0f;
    const float mx = m[0], my = m[1], xx = m[2], yy = m[3], xy = m[4];
    const float vx = fabsf(fmaf(-mx, mx, xx));
    const float vy = fabsf(fmaf(-my, my, yy));
    const float cxy = fmaf(-mx, my, xy);
    const float sdx = hw_sqrt(vx), sdy = hw_sqrt(vy);
    const float ux = mx + kMomentOffset, uy = my + kMomentOffset;
    const float dm = mx - my, ds = sdx - sdy;
    const float d1 = fmaf(ux, ux, fmaf(uy, uy, kC1));
    const float d2 = (vx + vy) + kC2;
    const float d3 = fmaf(sdx, sdy, kC3);
    const float d12 = d1 * d2;
    const float r = rcp(d12 * d3) * 0x1p24f;
    const float d3r = d3 * r;  // 2^24 / (d1 d2), shared by the first two quotients
    a.dl += (int)(((dm * dm) * d2) * d3r);
    a.dc += (int)(((ds * ds) * d1) * d3r);
    a.s += (int)((cxy + kC3) * (d12 * r));
}

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

    // A thread's few pixels (at most 64, so the integer sums fit 32 bits),
    // then the workgroup in fp64, exactly.
    LcsAcc acc;
    int npx = 0;
    vertical_moments<TW, TH, NT, RB, kNP>(lds, taps, x0, y0, MW, MH, [&](int, int, const float (&m)[kNP]) {
        ms_pixel(m, acc);
        ++npx;
    });
    double terms[3] = {(double)npx * 0x1p24 - acc.dl, (double)npx * 0x1p24 - acc.dc, (double)acc.s};
    block_sum<NT, 3>(terms, red);
    if (threadIdx.x == 0) {
        const int nb = gridDim.x * gridDim.y;
        const int slot = by * gridDim.x + bx;
        t.partials[slot] = terms[0];
        t.partials[nb + slot] = terms[1];
        t.partials[2 * nb + slot] = terms[2];
    }
}

// ------------------------------------------------------------ row streaming
//
// The level kernel above stages a 2-D tile and filters it horizontally over
// its 10-row halo too, so 16 % of its horizontal work is repeated by the tile
// below, and its moment planes make a round trip through LDS.  This kernel
// walks a strip down the plane instead: each thread owns two adjacent map
// columns, takes one input row at a time, filters it horizontally from a
// shared row buffer, and adds it into the eleven unfinished outputs of its
// columns held in registers (output j = t - 10 is complete after input row
// t).  Only the strip's top and bottom edges repeat work, (R + 10) / R.  The
// moments are bit-identical to the tile kernel's: the same products, and
// both 11-tap sums in the order k = 0..10.
//
// Workgroup: NW waves, a strip of 128 NW map columns and up
// to R map rows (R even, so the strip starts on an even row and the next
// level's 2x2 blocks do not straddle strips).  The row buffer holds the five
// per-sample planes x, y, x^2, y^2, xy of the strip's 128 NW + 10 input
// columns; it is double-buffered (a buffer is rewritten two rows later,
// after the row between has been read).  The first ten threads also convert
// the ten columns past the strip, for two rows at a time (four row buffers
// would let them take four, but their base registers cost the kernel its
// third wave per SIMD).  One wave per workgroup (kRowsWaves) measured fastest: it
// needs no barrier, only its own LDS accesses in order (wave_lds_order),
// which outweighs the halo columns costing the wave a second conversion pass
// (2160p MS-SSIM 19.6k frames/s against 19.0k with two waves and 17.0k with
// three, when each row still took a workgroup barrier).
//
// Loads and stores go through buffer resources whose row offset is a scalar,
// so a row costs no per-lane address arithmetic; columns past the plane are
// clamped to its last column (they feed only map columns outside the valid
// region, or no output at all), and rows never leave the plane.
constexpr unsigned kRsrcWord3 = 0x00020000;  // raw buffer, gfx9 family
constexpr int kRowsWaves = 1;                // waves per workgroup (strips of 128 kRowsWaves columns)

// A thread's two adjacent samples come from one load (load2) when the
// planes allow it (kPair), else from one load each.  values() gives the two
// samples' values from the loaded words w0, w1 (one load each: the two
// samples; one load: the packed pair in w0, or both words for fp32).
template <typename TIn> struct RowRaw;
template <> struct RowRaw<uint8_t> {
    __device__ static uint32_t load(__amdgpu_buffer_rsrc_t r, int vo, int so) {
        return __builtin_amdgcn_raw_buffer_load_b8(r, vo, so, 0);
    }
    __device__ static void load2(__amdgpu_buffer_rsrc_t r, int vo, int so, uint32_t &w0, uint32_t &w1) {
        w0 = __builtin_amdgcn_raw_buffer_load_b16(r, vo, so, 0);
        w1 = 0;
    }
    // Each byte of a pair converts in one instruction: the compiler takes
    // v_cvt_f32_ubyte0 for the low one, and the high one is written out
    // (knowing the load cleared bits 16-31, the compiler would shift first).
    template <bool kPair> __device__ static void values(uint32_t w0, uint32_t w1, float &a, float &b) {
        if constexpr (kPair) {
            a = (float)(w0 & 0xffu);
            asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(b) : "v"(w0));
        } else {
            a = (float)w0;
            b = (float)w1;
        }
    }
};
template <> struct RowRaw<uint16_t> {
    __device__ static uint32_t load(__amdgpu_buffer_rsrc_t r, int vo, int so) {
        return __builtin_amdgcn_raw_buffer_load_b16(r, vo, so, 0);
    }
    __device__ static void load2(__amdgpu_buffer_rsrc_t r, int vo, int so, uint32_t &w0, uint32_t &w1) {
        w0 = __builtin_amdgcn_raw_buffer_load_b32(r, vo, so, 0);
        w1 = 0;
    }
    template <bool kPair> __device__ static void values(uint32_t w0, uint32_t w1, float &a, float &b) {
        a = kPair ? (float)(w0 & 0xffffu) : (float)w0;
        b = kPair ? (float)(w0 >> 16) : (float)w1;
    }
};
template <> struct RowRaw<float> {
    __device__ static uint32_t load(__amdgpu_buffer_rsrc_t r, int vo, int so) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, vo, so, 0);
    }
    __device__ static void load2(__amdgpu_buffer_rsrc_t r, int vo, int so, uint32_t &w0, uint32_t &w1) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, vo, so, 0);
        w0 = v[0];
        w1 = v[1];
    }
    template <bool kPair> __device__ static void values(uint32_t w0, uint32_t w1, float &a, float &b) {
        a = __builtin_bit_cast(float, w0);
        b = __builtin_bit_cast(float, w1);
    }
};

// The raw samples of one input row that a thread converts: its two columns
// of both planes.
struct RowPair {
    uint32_t ra, rb, da, db;
};

// Orders a one-wave workgroup's LDS accesses as written.  The LDS performs
// one wave's accesses in issue order, so a row's reads see the writes issued
// before them without waiting for those writes to complete (the workgroup
// barrier's fence would: s_waitcnt lgkmcnt(0)); a wavefront-scope fence only
// keeps the compiler from moving accesses across it.
__device__ __forceinline__ void wave_lds_order() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

template <int... U, typename F>
__device__ __forceinline__ void static_steps(std::integer_sequence<int, U...>, F &&f) {
    (f(std::integral_constant<int, U>{}), ...);
}

template <typename TIn, int NW, bool kPair>
__global__ __launch_bounds__(64 * NW) void ms_level_rows(MsBatch b, int pitch, int W, int H, int next_pitch,
                                                         float unit, int R, Taps taps) {
    using Raw = RowRaw<TIn>;
    constexpr int S = 128 * NW;   // map columns of the strip, two per thread
    constexpr int P = S + 12;     // LDS row pitch: >= S + 10 floats, a multiple of 4
    __shared__ __attribute__((aligned(16))) float lds[2 * 5 * P];
    __shared__ double red[3][NW];

    int bx, by, bz;
    xcd_block(bx, by, bz);
    const MsFrame &fr = b.f[bz];
    const int MW = W - 10, MH = H - 10;
    const int x0 = bx * S, y0 = by * R;
    const int tid = threadIdx.x, c = 2 * tid;
    const bool last_x = bx == (int)gridDim.x - 1, last_y = by == (int)gridDim.y - 1;
    const int out_rows = min(R, MH - y0);     // map rows of this strip
    const int in_rows = min(R + 10, H - y0);  // input rows it reads

    const int nbytes = pitch * H * (int)sizeof(TIn);  // below 2^31 (checked by the launcher)
    const __amdgpu_buffer_rsrc_t rref = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(fr.ref), 0, nbytes,
                                                                          kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rdis = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(fr.dis), 0, nbytes,
                                                                          kRsrcWord3);
    const int row_bytes = pitch * (int)sizeof(TIn);
    const int voA = min(x0 + c, W - 1) * (int)sizeof(TIn), voB = min(x0 + c + 1, W - 1) * (int)sizeof(TIn);
    // A pair starts on an even column: past the plane it is the last pair
    // that starts inside it, whose values reach only map columns outside the
    // valid region (as does a pair's second sample past an odd width).
    const int last_pair = (W - 1) & ~1;
    const int voP = min(x0 + c, last_pair) * (int)sizeof(TIn);
    // The ten columns past the strip, for two rows at once: threads 0-4 take
    // the even row t of a pair, threads 5-9 the odd row t + 1, two columns
    // each, so the pass runs every other row.  (One wave: a row's buffer is
    // written one step early, after the wave has read the row it held.)
    static_assert(NW == 1, "the paired halo rows need a one-wave workgroup");
    const int hl = tid % 5, hr = tid < 10 ? tid / 5 : 0;
    const bool halo = tid < 10;
    const int hc = S + 2 * hl;  // strip-local first column of the halo thread's pair
    const int hvoA = min(x0 + hc, W - 1) * (int)sizeof(TIn);
    const int hvoB = min(x0 + hc + 1, W - 1) * (int)sizeof(TIn);
    const int hvoP = min(x0 + hc, last_pair) * (int)sizeof(TIn);

    auto load_row = [&](int t, RowPair &m) __attribute__((always_inline)) {
        const int so = (y0 + t) * row_bytes;
        if constexpr (kPair) {
            Raw::load2(rref, voP, so, m.ra, m.rb);
            Raw::load2(rdis, voP, so, m.da, m.db);
        } else {
            m.ra = Raw::load(rref, voA, so);
            m.rb = Raw::load(rref, voB, so);
            m.da = Raw::load(rdis, voA, so);
            m.db = Raw::load(rdis, voB, so);
        }
    };
    // Halo samples of the row pair (t, t + 1), t even; without a row t + 1
    // the odd threads read row t again (and their values go unused).
    auto load_halo = [&](int t, RowPair &h) __attribute__((always_inline)) {
        const int so = (y0 + t) * row_bytes;
        const int dr = (hr != 0 && t + 1 < in_rows) ? row_bytes : 0;
        if constexpr (kPair) {
            Raw::load2(rref, hvoP + dr, so, h.ra, h.rb);
            Raw::load2(rdis, hvoP + dr, so, h.da, h.db);
        } else {
            h.ra = Raw::load(rref, hvoA + dr, so);
            h.rb = Raw::load(rref, hvoB + dr, so);
            h.da = Raw::load(rdis, hvoA + dr, so);
            h.db = Raw::load(rdis, hvoB + dr, so);
        }
    };

    // Next level: this thread's 2x2 block column, and (last strip only) the
    // halo threads' ones; a block row is complete at each odd input row.
    float *const nref = fr.next_ref;
    const bool has_next = nref != nullptr;
    const int nW = W / 2, nH = H / 2;
    const int nbx = (x0 + c) / 2, hnbx = (x0 + hc) / 2;
    const bool own_x = nbx < nW, hown_x = last_x && tid < 5 && hnbx < nW;
    // (At the last level there is no next plane: the resources then cover
    // nothing and no store is issued.)
    const int nbytes_next = has_next ? next_pitch * nH * 4 : 0;
    const __amdgpu_buffer_rsrc_t nr = __builtin_amdgcn_make_buffer_rsrc(nref, 0, nbytes_next, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t nd = __builtin_amdgcn_make_buffer_rsrc(fr.next_dis, 0, nbytes_next, kRsrcWord3);

    float ring[11][5][2];  // the eleven unfinished outputs of the thread's two columns
#pragma unroll
    for (int s = 0; s < 11; ++s)
#pragma unroll
        for (int p = 0; p < 5; ++p) ring[s][p][0] = ring[s][p][1] = 0.0f;

    // The terms of both columns are formed and added unconditionally, into
    // an accumulator per column (at most 22 pixels, one group of rows, in
    // 32-bit integers), so the two pixels' dependency chains interleave; a
    // column outside the valid map region (its inputs are clamped, so its
    // terms are finite) is dropped once per group.
    const bool vA = x0 + c < MW, vB = x0 + c + 1 < MW;
    LcsAcc accA, accB;
    double DL = 0.0, DC = 0.0, PS = 0.0;
    float psx = 0.0f, psy = 0.0f;  // the previous row's pair sums

    // Byte offsets in LDS of the thread's first column in each row buffer
    // and in that buffer's last plane, kept in registers of their own (the
    // empty asm hides their values from the compiler): every read and write
    // of a row then takes a constant below 2040 bytes, which the 8-bit offset
    // fields of paired LDS accesses hold, instead of an address addition per
    // access.  plane_at(u & 1, p) is plane p of row t's buffer (t0 is even).
    int lofs[2][2] = {{4 * c, 4 * (c + 4 * P)}, {4 * (c + 5 * P), 4 * (c + 9 * P)}};
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) asm volatile("" : "+v"(lofs[i][j]));
    auto plane_at = [&](int parity, int p) __attribute__((always_inline)) {
        return p < 4 ? reinterpret_cast<float *>(reinterpret_cast<char *>(lds) + lofs[parity][0]) + p * P
                     : reinterpret_cast<float *>(reinterpret_cast<char *>(lds) + lofs[parity][1]);
    };

    RowPair nm{}, nh{};
    load_row(0, nm);
    load_halo(0, nh);
    // Groups of 22 rows: the eleven output slots and the row buffer's parity
    // are compile-time at every step (22 rows unrolled against 11 issue 6 %
    // fewer VALU instructions; level 1 at 2160p 1093 -> 1080 us per batch).
    for (int t0 = 0; t0 < in_rows; t0 += 22) {
        static_steps(std::make_integer_sequence<int, 22>{}, [&](auto uc) __attribute__((always_inline)) {
            constexpr int u = decltype(uc)::value;
            const int t = t0 + u;
            if (t >= in_rows) return;
            // Convert this row, then reuse its registers for the next row's
            // loads (they land while this row is filtered).
            float va, vb, wa, wb;
            Raw::template values<kPair>(nm.ra, nm.rb, va, vb);
            Raw::template values<kPair>(nm.da, nm.db, wa, wb);
            const float xa = fmaf(va, unit, -kMomentOffset), xb = fmaf(vb, unit, -kMomentOffset);
            const float ya = fmaf(wa, unit, -kMomentOffset), yb = fmaf(wb, unit, -kMomentOffset);
            *reinterpret_cast<float2 *>(plane_at(u & 1, 0)) = make_float2(xa, xb);
            *reinterpret_cast<float2 *>(plane_at(u & 1, 1)) = make_float2(ya, yb);
            *reinterpret_cast<float2 *>(plane_at(u & 1, 2)) = make_float2(xa * xa, xb * xb);
            *reinterpret_cast<float2 *>(plane_at(u & 1, 3)) = make_float2(ya * ya, yb * yb);
            *reinterpret_cast<float2 *>(plane_at(u & 1, 4)) = make_float2(xa * ya, xb * yb);
            // Next level: the block row (t - 1, t) when t is odd.
            const bool block_row = has_next && (t & 1) != 0 && (t - 1 < R || last_y);
            const int so_next = ((y0 + t) / 2) * next_pitch * 4;
            const float sx = xa + xb, sy = ya + yb;
            if (block_row && own_x) {
                __builtin_amdgcn_raw_buffer_store_b32(
                    __builtin_bit_cast(uint32_t, fmaf(psx + sx, 0.25f, kMomentOffset)), nr, nbx * 4, so_next, 0);
                __builtin_amdgcn_raw_buffer_store_b32(
                    __builtin_bit_cast(uint32_t, fmaf(psy + sy, 0.25f, kMomentOffset)), nd, nbx * 4, so_next, 0);
            }
            if ((u & 1) == 0) {
                psx = sx;  // the next (odd) row's block row pairs with this row
                psy = sy;
                // Row t + 1's halo goes into the buffer the previous row was
                // read from: those reads come first.
                wave_lds_order();
                if (halo) {
                    float hva, hvb, hwa, hwb;
                    Raw::template values<kPair>(nh.ra, nh.rb, hva, hvb);
                    Raw::template values<kPair>(nh.da, nh.db, hwa, hwb);
                    const float hxa = fmaf(hva, unit, -kMomentOffset), hxb = fmaf(hvb, unit, -kMomentOffset);
                    const float hya = fmaf(hwa, unit, -kMomentOffset), hyb = fmaf(hwb, unit, -kMomentOffset);
                    float *hb = lds + ((t + hr) & 1) * 5 * P;  // row t, or row t + 1's buffer
                    *reinterpret_cast<float2 *>(hb + 0 * P + hc) = make_float2(hxa, hxb);
                    *reinterpret_cast<float2 *>(hb + 1 * P + hc) = make_float2(hya, hyb);
                    *reinterpret_cast<float2 *>(hb + 2 * P + hc) = make_float2(hxa * hxa, hxb * hxb);
                    *reinterpret_cast<float2 *>(hb + 3 * P + hc) = make_float2(hya * hya, hyb * hyb);
                    *reinterpret_cast<float2 *>(hb + 4 * P + hc) = make_float2(hxa * hya, hxb * hyb);
                    // Next level: the block row (t, t + 1) of the halo
                    // columns (the plane's last strip only, a wave-uniform
                    // test), the odd row's pair sums from thread + 5.
                    if (has_next && last_x && (t < R || last_y) && t + 1 < in_rows) {
                        const float hsx = hxa + hxb, hsy = hya + hyb;
                        const float osx = __builtin_bit_cast(
                            float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, hsx), 0x105, 0xF, 0xF, false));
                        const float osy = __builtin_bit_cast(
                            float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, hsy), 0x105, 0xF, 0xF, false));
                        if (hown_x) {
                            const int so_h = ((y0 + t) / 2) * next_pitch * 4;
                            __builtin_amdgcn_raw_buffer_store_b32(
                                __builtin_bit_cast(uint32_t, fmaf(hsx + osx, 0.25f, kMomentOffset)), nr, hnbx * 4,
                                so_h, 0);
                            __builtin_amdgcn_raw_buffer_store_b32(
                                __builtin_bit_cast(uint32_t, fmaf(hsy + osy, 0.25f, kMomentOffset)), nd, hnbx * 4,
                                so_h, 0);
                        }
                    }
                }
                if (t + 2 < in_rows) load_halo(t + 2, nh);
            }
            if (t + 1 < in_rows) load_row(t + 1, nm);

            wave_lds_order();  // the row is in the buffer

            // Horizontal 11-tap sums of the thread's two columns, plane by
            // plane, each added at once into the eleven unfinished outputs.
#pragma unroll
            for (int p = 0; p < 5; ++p) {
                float v[12];
#pragma unroll
                for (int k = 0; k < 6; ++k) {
                    const float2 w = *reinterpret_cast<const float2 *>(plane_at(u & 1, p) + 2 * k);
                    v[2 * k] = w.x;
                    v[2 * k + 1] = w.y;
                }
                float h0 = 0.0f, h1 = 0.0f;
#pragma unroll
                for (int k = 0; k < 11; ++k) {
                    h0 = fmaf(taps.g[k], v[k], h0);
                    h1 = fmaf(taps.g[k], v[k + 1], h1);
                }
#pragma unroll
                for (int s = 0; s < 11; ++s) {
                    const int k = (u - s + 11) % 11;  // this row's tap for the output in slot s
                    if (k == 0) {
                        ring[s][p][0] = fmaf(taps.g[0], h0, 0.0f);
                        ring[s][p][1] = fmaf(taps.g[0], h1, 0.0f);
                    } else {
                        ring[s][p][0] = fmaf(taps.g[k], h0, ring[s][p][0]);
                        ring[s][p][1] = fmaf(taps.g[k], h1, ring[s][p][1]);
                    }
                }
            }

            // Output t - 10 is complete; it sits in slot (u + 1) % 11.
            const int j = t - 10;
            if (j >= 0 && j < out_rows) {
                constexpr int sc = (u + 1) % 11;
                const float ma[5] = {ring[sc][0][0], ring[sc][1][0], ring[sc][2][0], ring[sc][3][0],
                                     ring[sc][4][0]};
                const float mb[5] = {ring[sc][0][1], ring[sc][1][1], ring[sc][2][1], ring[sc][3][1],
                                     ring[sc][4][1]};
                ms_pixel(ma, accA);
                ms_pixel(mb, accB);
            }
        });
        DL += (double)(vA ? accA.dl : 0) + (double)(vB ? accB.dl : 0);
        DC += (double)(vA ? accA.dc : 0) + (double)(vB ? accB.dc : 0);
        PS += (double)(vA ? accA.s : 0) + (double)(vB ? accB.s : 0);
        accA = LcsAcc{};
        accB = LcsAcc{};
    }

    const double npx = (double)out_rows * (double)((int)vA + (int)vB) * 0x1p24;
    double terms[3] = {npx - DL, npx - DC, PS};
    block_sum<64 * NW, 3>(terms, red);
    if (tid == 0) {
        const int nb = gridDim.x * gridDim.y;
        const int slot = by * gridDim.x + bx;
        fr.partials[slot] = terms[0];
        fr.partials[nb + slot] = terms[1];
        fr.partials[2 * nb + slot] = terms[2];
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
            lcs[j] = tot[0] / lv.count[j] * 0x1p-24;
            lcs[5 + j] = tot[1] / lv.count[j] * 0x1p-24;
            lcs[10 + j] = tot[2] / lv.count[j] * 0x1p-24;
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
    if ((b.lcs_mask >> blockIdx.x) & 1u)
        for (int j = 0; j < 15; ++j) fr.result[1 + j] = lcs[j];
    __threadfence_system();
}

// Which level kernel a batch takes, and its grid.  The choice compares
// estimates of the VALU issue each needs per SIMD (256 CUs x 4 SIMDs), from
// the instruction counts of their compiled code: the tile kernel issues about
// 914 VALU instructions per wave, spread over the whole chip; the row kernel
// about 330 per wave and input row, and it runs in rounds of three waves per
// SIMD (its register use allows three), each round as long as its strips are
// tall.  So the row kernel wins on large planes in large batches (2160p
// levels 1-3 in batches of 32), and the tile kernel on small planes or
// batches, whose few tall strips would leave most SIMDs idle.  The strip
// height R (even, at least 16 rows) is picked by the same estimate: 136 rows
// (five rounds) at 2160p level 1 and 180 rows (one round) at level 2 in
// batches of 32, which a sweep of R on the hardware also found best.  The row
// kernel's buffer offsets are 32-bit, so planes of 2^31 bytes or more (fp32
// levels, pitch up to W + 63) always take the tile kernel.
struct MsPlan {
    bool rows;
    int R, gx, gy;  // strip height (row kernel) and grid
};

constexpr double kTileWaveInstr = 914.0, kRowsStepInstr = 330.0;
constexpr int kSimds = 256 * 4, kRowsWavesPerSimd = 3, kRowsMinR = 16;
// A plan's rounds cost a tenth of a round more, for the spread of its
// strips' finishing times: measured at 2160p (batches of 32), strips of
// 120-136 rows in five rounds run 8 % faster than strips of 718 rows in one
// round that leaves 6 % of the slots empty, which the bare count calls even.
constexpr double kRowsTail = 0.1;

// The best plan by the estimate above; `fractional`: a partly filled last
// round costs only its share of a round.
MsPlan ms_plan_by(int W, int H, int n, bool fractional) {
    const int MW = W - 10, MH = H - 10;
    MsPlan p{false, 0, (MW + kTW - 1) / kTW, (MH + kTH - 1) / kTH};
    if ((long long)(W + 64) * (long long)H * 4 >= (1ll << 31)) return p;
    double best = kTileWaveInstr * (kNT / 64) * (double)p.gx * (double)p.gy * n / kSimds;
    const long long slots = (long long)kRowsWavesPerSimd * kSimds;
    const int gx = (MW + 128 * kRowsWaves - 1) / (128 * kRowsWaves);
    for (int strips = 1; strips <= MH / kRowsMinR; ++strips) {
        int R = (MH + strips - 1) / strips;
        R += R & 1;
        const int gy = (MH + R - 1) / R;
        const long long waves = (long long)kRowsWaves * gx * gy * n;
        const double rounds =
            (fractional ? (double)waves / (double)slots : (double)((waves + slots - 1) / slots)) + kRowsTail;
        const double cost = rounds * kRowsWavesPerSimd * (R + 10) * kRowsStepInstr;
        if (cost < best) {
            best = cost;
            p = MsPlan{true, R, gx, gy};
        }
    }
    return p;
}

// An overlapped batch (another batch of its context runs on a second
// stream) leaves the idle slots of its strips' last round to the other
// batch's waves.  Where its plan alone runs several rounds of strips, it
// takes the plan that counts that last round fractionally: taller strips,
// less halo (2160p level 1 in batches of 32: 308-row strips in 2.2 rounds
// instead of 136 rows in 5, 21.9k -> 22.4k frames/s on one context; alone
// they would cost 4 %).  A level whose plan alone fits one round keeps it:
// re-planned (2160p levels 2 and 3: 134 and 76 rows instead of 180 and 46)
// it measured slower, 20.8k with level 1 re-planned too.
MsPlan ms_plan(int W, int H, int n, bool overlapped) {
    const MsPlan alone = ms_plan_by(W, H, n, false);
    if (!overlapped || !alone.rows) return alone;
    const long long waves = (long long)kRowsWaves * alone.gx * alone.gy * n;
    if (waves <= (long long)kRowsWavesPerSimd * kSimds) return alone;
    return ms_plan_by(W, H, n, true);
}

}  // namespace

int ms_partials(int W, int H, int n, bool overlapped) {
    const MsPlan p = ms_plan(W, H, n, overlapped);
    return p.gx * p.gy;
}

int ms_partials_max(int W, int H) {
    int m = 0;
    for (int n = 1; n <= kMaxBatch; ++n)
        m = std::max(m, std::max(ms_partials(W, H, n, false), ms_partials(W, H, n, true)));
    return m;
}

template <typename TIn>
hipError_t launch_rows(const MsPlan &p, const MsBatch &b, int n, int pitch, int W, int H, int next_pitch,
                       float unit, const Taps &taps, hipStream_t stream, const KernelTimer &timer) {
    const dim3 grid(p.gx, p.gy, n);
    // Pair loads need every row of every plane to start on a pair boundary.
    bool pair = pitch % 2 == 0;
    for (int i = 0; i < n; ++i)
        if (((uintptr_t)b.f[i].ref | (uintptr_t)b.f[i].dis) % (2 * sizeof(TIn)) != 0) pair = false;
    if (pair)
        return launch_kernel(ms_level_rows<TIn, kRowsWaves, true>, grid, dim3(64 * kRowsWaves), stream, timer, b,
                             pitch, W, H, next_pitch, unit, p.R, taps);
    return launch_kernel(ms_level_rows<TIn, kRowsWaves, false>, grid, dim3(64 * kRowsWaves), stream, timer, b, pitch,
                         W, H, next_pitch, unit, p.R, taps);
}

hipError_t launch_ms_level(const MsBatch &b, int n, InKind kind, int pitch, int W, int H, int next_pitch,
                           float unit, const Taps &taps, bool overlapped, hipStream_t stream,
                           const KernelTimer &timer) {
    if (n < 1 || n > kMaxBatch) return hipErrorInvalidValue;
    const MsPlan p = ms_plan(W, H, n, overlapped);
    const dim3 grid(p.gx, p.gy, n);
    if (p.rows) {
        switch (kind) {
        case IN_F32:
            return launch_rows<float>(p, b, n, pitch, W, H, next_pitch, unit, taps, stream, timer);
        case IN_U8:
            return launch_rows<uint8_t>(p, b, n, pitch, W, H, next_pitch, unit, taps, stream, timer);
        case IN_U16:
            return launch_rows<uint16_t>(p, b, n, pitch, W, H, next_pitch, unit, taps, stream, timer);
        default:
            return hipErrorInvalidValue;
        }
    }
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
