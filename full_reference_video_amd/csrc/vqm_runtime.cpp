// vqm_runtime.cpp — the C ABI of include/vqm.h: argument checks and the gate,
// contexts with a FIFO of in-flight frame slots, one upload per frame, the
// kernel launches, the one wait per frame, and the last-error message.
//
// "ADR-1405: float_ssim_hip decimates on the device, bit-identical to the
// CPU", Decision 4: the gate refuses only what the method does not define
// (scale > 128, decimated plane below 11 x 11) and runs on the host before
// any HIP call.  "Research-1369: SYCL psnr_hvs, motion_v2 and psnr at 4K",
// §4–§5 and §7: pageable input goes through pinned staging with one DMA per
// plane; a slot is reused only after the frame that used it was collected
// (so no upload overwrites data a kernel still reads); scratch is keyed by
// the frame geometry and rebuilt when it changes.
#include "vqm.h"

#include <errno.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <cmath>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <deque>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "msssim_kernels.h"
#include "probe.h"
#include "ss2_kernels.h"
#include "vqm_kernels.h"

static_assert(VQM_MAX_BATCH == vqm::kMaxBatch, "batch limits of the ABI and the kernels differ");

namespace {

thread_local std::string g_err;

int fail(int rc, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return rc;
}

#define HIP_TRY(call)                                                                              \
    do {                                                                                           \
        hipError_t e_ = (call);                                                                    \
        if (e_ != hipSuccess) return fail(-EIO, "%s: %s", #call, hipGetErrorString(e_));           \
    } while (0)

#define HIP_TRY_ALLOC(call)                                                                        \
    do {                                                                                           \
        hipError_t e_ = (call);                                                                    \
        if (e_ == hipErrorOutOfMemory || e_ == hipErrorMemoryAllocation)                           \
            return fail(-ENOMEM, "%s: %s", #call, hipGetErrorString(e_));                          \
        if (e_ != hipSuccess) return fail(-EIO, "%s: %s", #call, hipGetErrorString(e_));           \
    } while (0)

enum Kind { KIND_NONE = 0, KIND_SSIM = 1, KIND_MSSSIM = 2 };

constexpr int kLevels = 5;
constexpr int kWin = 11;

int scale_of(int w, int h) {
    const int m = w < h ? w : h;
    const int s = (int)round((double)m / 256.0);
    return s < 1 ? 1 : s;
}

int check_args(const void *ref, const void *dis, int w, int h, int bpc) {
    if (!ref || !dis) return fail(-EINVAL, "NULL plane pointer");
    if (w <= 0 || h <= 0) return fail(-EINVAL, "frame size %dx%d is not positive", w, h);
    if ((long long)w * (long long)h > 0x7fffffffLL) return fail(-EINVAL, "frame %dx%d too large", w, h);
    if (bpc < 8 || bpc > 16) return fail(-EINVAL, "bpc %d outside 8..16", bpc);
    return 0;
}

int gate_ssim(int w, int h, int bpc, int *s_out, int *dw_out, int *dh_out) {
    if (w <= 0 || h <= 0) return fail(-EINVAL, "frame size %dx%d is not positive", w, h);
    if ((long long)w * (long long)h > 0x7fffffffLL) return fail(-EINVAL, "frame %dx%d too large", w, h);
    if (bpc < 8 || bpc > 16) return fail(-EINVAL, "bpc %d outside 8..16", bpc);
    const int s = scale_of(w, h);
    const int dw = (w + s - 1) / s, dh = (h + s - 1) / s;
    if (s > 128) return fail(-ENOTSUP, "float_ssim: scale %d exceeds 128 for %dx%d", s, w, h);
    if (dw < kWin || dh < kWin)
        return fail(-ENOTSUP, "float_ssim: decimated plane %dx%d is smaller than the 11x11 window", dw, dh);
    if (s_out) *s_out = s;
    if (dw_out) *dw_out = dw;
    if (dh_out) *dh_out = dh;
    return 0;
}

int gate_msssim(int w, int h) {
    if (w / 16 < kWin || h / 16 < kWin)
        return fail(-ENOTSUP, "MS-SSIM: level 5 of %dx%d (%dx%d) is smaller than the 11x11 window", w, h,
                    w / 16, h / 16);
    return 0;
}

int round_up(int v, int m) { return (v + m - 1) / m * m; }

// Normalised 11-tap Gaussian, sigma 1.5, rounded to fp32.
vqm::Taps make_taps() {
    double g[11], sum = 0.0;
    for (int k = 0; k < 11; ++k) {
        const double d = k - 5;
        g[k] = exp(-d * d / (2.0 * 1.5 * 1.5));
        sum += g[k];
    }
    vqm::Taps t;
    for (int k = 0; k < 11; ++k) t.g[k] = (float)(g[k] / sum);
    return t;
}

struct Geometry {
    int kind = KIND_NONE, w = 0, h = 0, bpc = 0;
    int s = 1, dw = 0, dh = 0, dpitch = 0;         // float_ssim
    int lw[kLevels] = {}, lh[kLevels] = {}, lpitch[kLevels] = {};  // MS-SSIM
    bool operator==(const Geometry &o) const {
        return kind == o.kind && w == o.w && h == o.h && bpc == o.bpc && s == o.s;
    }
    size_t sample_bytes() const { return bpc == 8 ? 1 : 2; }
    size_t plane_bytes() const { return (size_t)w * (size_t)h * sample_bytes(); }
};

Geometry make_geometry(int kind, int w, int h, int bpc) {
    Geometry g;
    g.kind = kind;
    g.w = w;
    g.h = h;
    g.bpc = bpc;
    if (kind == KIND_SSIM) {
        g.s = scale_of(w, h);
        g.dw = (w + g.s - 1) / g.s;
        g.dh = (h + g.s - 1) / g.s;
        g.dpitch = round_up(g.dw, 64);
    } else {
        int lw = w, lh = h;
        for (int j = 0; j < kLevels; ++j) {
            g.lw[j] = lw;
            g.lh[j] = lh;
            g.lpitch[j] = j == 0 ? w : round_up(lw, 64);
            lw /= 2;
            lh /= 2;
        }
    }
    return g;
}

// Device scratch and host result slot of one frame in flight.
struct Slot {
    Geometry geo;
    void *dev_in = nullptr;         // device copy of host input: ref then dis
    size_t dev_in_bytes = 0;
    void *staging = nullptr;        // pinned host staging for pageable input
    size_t staging_bytes = 0;
    float *planes = nullptr;        // decimated planes or pyramid levels 2..5
    size_t planes_bytes = 0;
    double *partials = nullptr;
    size_t partials_count = 0;
    double *result_host = nullptr;  // pinned: score + 15 means
    double *result_dev = nullptr;   // its device-visible address
    bool ready = false;             // scratch allocated for geo
    struct BatchEvent *batch = nullptr;  // completion of the batch this frame rode in
    int kind = KIND_NONE;
    bool extra = false;             // the finish also writes the dB form / the 15 level means

    // offsets (in floats) of the planes inside `planes`
    size_t off_ref[kLevels] = {}, off_dis[kLevels] = {};
    size_t span[kLevels] = {};      // partials offset of each MS level

    void release() {
        if (dev_in) (void)hipFree(dev_in);
        if (staging) (void)hipHostFree(staging);
        if (planes) (void)hipFree(planes);
        if (partials) (void)hipFree(partials);
        if (result_host) (void)hipHostFree(result_host);
        *this = Slot();
    }
};

// One completion event per submitted batch, shared by the batch's frames:
// the first collect of the batch waits on it, the others find it done.  It
// returns to the pool when its last frame is collected.
struct BatchEvent {
    hipEvent_t ev = nullptr;
    int refs = 0;
    bool completed = false;
};

// A float_ssim batch inside the step pipeline.
enum Stage { STAGE_DECIMATED = 0, STAGE_MAPPED = 1 };
struct PendingBatch {
    Slot *sl[VQM_MAX_BATCH];
    const void *in_r[VQM_MAX_BATCH], *in_d[VQM_MAX_BATCH];  // device-readable raw planes
    int n = 0;
    int stage = STAGE_DECIMATED;  // the last stage a launch already enqueued for it
};

struct TimedLaunch {
    hipEvent_t start, stop;
    int cls;
    int frames;
};

}  // namespace

// A ssimulacra2 chain's device workspace and its pinned result block.
struct Ss2Buffers {
    float *work = nullptr;
    size_t work_floats = 0;
    double *res_host = nullptr, *res_dev = nullptr;
    void release() {
        if (work) (void)hipFree(work);
        if (res_host) (void)hipHostFree(res_host);
        work = nullptr;
        res_host = res_dev = nullptr;
        work_floats = 0;
    }
};

// A submitted chain frame: its buffers, its own stream (so frames in flight
// overlap on the GPU), an event ordering it after the context's stream, and
// its completion event.
struct Ss2Slot {
    Ss2Buffers buf;
    hipStream_t stream = nullptr;
    hipEvent_t ready = nullptr, done = nullptr;
    int nres = 0;
    void release() {
        if (stream) {
            (void)hipStreamSynchronize(stream);
            (void)hipStreamDestroy(stream);
        }
        if (ready) (void)hipEventDestroy(ready);
        if (done) (void)hipEventDestroy(done);
        stream = nullptr;
        ready = done = nullptr;
        buf.release();
    }
};

struct vqm_ctx {
    int device = 0;
    hipStream_t stream = nullptr;
    bool own_stream = false;
    vqm::Taps taps;
    Slot slots[VQM_MAX_IN_FLIGHT];
    int head = 0, count = 0;
    std::vector<std::unique_ptr<BatchEvent>> batch_events;
    // float_ssim batches whose pipeline (decimate -> map -> finish, one stage
    // per step launch) has not finished yet, oldest first; same geometry.
    std::deque<PendingBatch> pipeline;
    bool timing = false;
    bool capturing = false;              // launches go into a graph: no completion events
    // MS-SSIM batches of a context that owns its stream alternate between
    // that stream and this one (made on first use), so that one batch's
    // small levels run beside the next batch's first level; `ms_ready`
    // orders a batch on ms_aux after the uploads on the context's stream.
    hipStream_t ms_aux = nullptr;
    hipEvent_t ms_ready = nullptr;
    bool ms_flip = false;
    bool ms_overlap = false;  // a caller's context on a library-owned stream (not the blocking calls' pool)
    std::vector<TimedLaunch> timed;      // recorded, not yet read
    std::vector<hipEvent_t> event_pool;  // free timing events
    double time_ms[4] = {0, 0, 0, 0};
    int launches[4] = {0, 0, 0, 0};
    int frames[4] = {0, 0, 0, 0};
    // ssimulacra2 statistics: workgroup partials and the pinned result block
    void *ss2_partials = nullptr;
    double *ss2_result_host = nullptr, *ss2_result_dev = nullptr;
    // ssimulacra2 per-scale chain of the blocking calls (the workspace and
    // the pinned block of every scale's sums), and the slots of frames
    // submitted on this context, each with its own stream
    Ss2Buffers ss2c;
    Ss2Slot ss2_slot[VQM_SS2_MAX_IN_FLIGHT];
    int ss2_head = 0, ss2_count = 0;
};

namespace {

// The caller's current device is theirs: an entry point that switches to a
// context's device switches back before it returns.  The outermost scope of
// a thread records the device ensure_device found, and only if it switched
// (so entry points still make no HIP call before their argument checks).
struct DeviceScope;
thread_local DeviceScope *t_scope = nullptr;
struct DeviceScope {
    int prev = -1;
    bool outer;
    DeviceScope() : outer(t_scope == nullptr) {
        if (outer) t_scope = this;
    }
    ~DeviceScope() {
        if (!outer) return;
        t_scope = nullptr;
        if (prev >= 0) (void)hipSetDevice(prev);
    }
    DeviceScope(const DeviceScope &) = delete;
    DeviceScope &operator=(const DeviceScope &) = delete;
};

int ensure_device(vqm_ctx *ctx) {
    int cur = -1;
    HIP_TRY(hipGetDevice(&cur));
    if (cur != ctx->device) {
        if (t_scope && t_scope->prev < 0) t_scope->prev = cur;
        HIP_TRY(hipSetDevice(ctx->device));
    }
    return 0;
}

// Size (or rebuild) a slot's scratch for geometry g.  The slot is idle.
int prepare_slot(Slot &sl, const Geometry &g) {
    if (sl.ready && sl.geo == g) return 0;
    sl.release();
    sl.geo = g;
    size_t floats = 0, partials = 0;
    if (g.kind == KIND_SSIM) {
        const size_t plane = (size_t)g.dpitch * (size_t)g.dh;
        sl.off_ref[0] = 0;
        sl.off_dis[0] = plane;
        floats = 2 * plane;
        partials = (size_t)vqm::ssim_partials(g.dw, g.dh);
    } else {
        for (int j = 1; j < kLevels; ++j) {
            const size_t plane = (size_t)g.lpitch[j] * (size_t)g.lh[j];
            sl.off_ref[j] = floats;
            sl.off_dis[j] = floats + plane;
            floats += 2 * plane;
        }
        for (int j = 0; j < kLevels; ++j) {
            sl.span[j] = partials;
            partials += 3 * (size_t)vqm::ms_partials_max(g.lw[j], g.lh[j]);
        }
    }
    sl.planes_bytes = floats * sizeof(float);
    HIP_TRY_ALLOC(hipMalloc(&sl.planes, sl.planes_bytes));
    sl.partials_count = partials;
    HIP_TRY_ALLOC(hipMalloc(&sl.partials, partials * sizeof(double)));
    HIP_TRY_ALLOC(hipHostMalloc(&sl.result_host, 16 * sizeof(double), hipHostMallocMapped | hipHostMallocCoherent));
    HIP_TRY(hipHostGetDevicePointer(reinterpret_cast<void **>(&sl.result_dev), sl.result_host, 0));
    sl.ready = true;
    return 0;
}

// Flags of the events the host waits on before it reads a batch's results.
// The results are the only memory the host reads after such a wait, and the
// finish roles write them to coherent pinned host memory followed by a
// system-scope fence of their own, so they are visible before the kernel
// ends; the event's own system-scope release (an L2 write-back of the
// decimated planes and partials, which the host never reads) is dropped:
// 1.2 % of the 2160p float_ssim stream.
constexpr unsigned kResultEventFlags = hipEventDisableTiming | hipEventDisableSystemFence;

// A free batch event (no frame of an earlier batch still refers to it).
int take_batch_event(vqm_ctx *ctx, BatchEvent **out) {
    for (auto &be : ctx->batch_events)
        if (be->refs == 0) {
            *out = be.get();
            return 0;
        }
    std::unique_ptr<BatchEvent> be(new BatchEvent());
    HIP_TRY(hipEventCreateWithFlags(&be->ev, kResultEventFlags));
    *out = be.get();
    ctx->batch_events.push_back(std::move(be));
    return 0;
}

enum PtrKind { PTR_PAGEABLE, PTR_PINNED, PTR_DEVICE };

int classify(const void *p, int device, PtrKind *out) {
    hipPointerAttribute_t a;
    memset(&a, 0, sizeof a);
    hipError_t e = hipPointerGetAttributes(&a, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();  // pageable memory is reported as an error
        *out = PTR_PAGEABLE;
        return 0;
    }
    switch (a.type) {
    case hipMemoryTypeDevice:
    case hipMemoryTypeManaged:
        if (a.device != device)
            return fail(-EINVAL, "plane is device memory of device %d, context is on %d", a.device, device);
        *out = PTR_DEVICE;
        return 0;
    case hipMemoryTypeHost:
        *out = PTR_PINNED;
        return 0;
    default:
        *out = PTR_PAGEABLE;
        return 0;
    }
}

// Make both planes readable by kernels on ctx's stream: device input is used
// in place; host input is sent with one DMA (pageable input is first copied
// into pinned staging, which is free because the slot is idle).
int upload(vqm_ctx *ctx, Slot &sl, const void *ref, const void *dis, const void **dref,
           const void **ddis) {
    PtrKind kr, kd;
    int rc = classify(ref, ctx->device, &kr);
    if (rc) return rc;
    rc = classify(dis, ctx->device, &kd);
    if (rc) return rc;
    if (kr == PTR_DEVICE && kd == PTR_DEVICE) {
        *dref = ref;
        *ddis = dis;
        return 0;
    }
    const size_t pb = sl.geo.plane_bytes();
    if (sl.dev_in_bytes < 2 * pb) {
        if (sl.dev_in) (void)hipFree(sl.dev_in);
        sl.dev_in = nullptr;
        sl.dev_in_bytes = 0;
        HIP_TRY_ALLOC(hipMalloc(&sl.dev_in, 2 * pb));
        sl.dev_in_bytes = 2 * pb;
    }
    char *din = static_cast<char *>(sl.dev_in);
    const void *src[2] = {ref, dis};
    const PtrKind kind[2] = {kr, kd};
    void *dst[2] = {din, din + pb};
    if (kr == PTR_PAGEABLE || kd == PTR_PAGEABLE) {
        if (sl.staging_bytes < 2 * pb) {
            if (sl.staging) (void)hipHostFree(sl.staging);
            sl.staging = nullptr;
            sl.staging_bytes = 0;
            HIP_TRY_ALLOC(hipHostMalloc(&sl.staging, 2 * pb, hipHostMallocDefault));
            sl.staging_bytes = 2 * pb;
        }
    }
    char *stg = static_cast<char *>(sl.staging);
    if (kr == PTR_PAGEABLE && kd == PTR_PAGEABLE) {
        memcpy(stg, ref, pb);
        memcpy(stg + pb, dis, pb);
        HIP_TRY(hipMemcpyAsync(din, stg, 2 * pb, hipMemcpyHostToDevice, ctx->stream));
    } else {
        for (int i = 0; i < 2; ++i) {
            if (kind[i] == PTR_DEVICE) {
                HIP_TRY(hipMemcpyAsync(dst[i], src[i], pb, hipMemcpyDeviceToDevice, ctx->stream));
            } else if (kind[i] == PTR_PINNED) {
                HIP_TRY(hipMemcpyAsync(dst[i], src[i], pb, hipMemcpyHostToDevice, ctx->stream));
            } else {
                memcpy(stg + i * pb, src[i], pb);
                HIP_TRY(hipMemcpyAsync(dst[i], stg + i * pb, pb, hipMemcpyHostToDevice, ctx->stream));
            }
        }
    }
    *dref = din;
    *ddis = din + pb;
    return 0;
}

// Events for one timed launch (taken from the pool); the launch itself
// records them at the kernel's start and end.
int timing_begin(vqm_ctx *ctx, TimedLaunch *tl, int cls, int frames, vqm::KernelTimer *kt) {
    if (!ctx->timing) return 0;
    for (int i = 0; i < 2; ++i) {
        hipEvent_t e;
        if (!ctx->event_pool.empty()) {
            e = ctx->event_pool.back();
            ctx->event_pool.pop_back();
        } else {
            HIP_TRY(hipEventCreate(&e));
        }
        (i == 0 ? tl->start : tl->stop) = e;
    }
    tl->cls = cls;
    tl->frames = frames;
    kt->start = tl->start;
    kt->stop = tl->stop;
    return 0;
}

void timing_end(vqm_ctx *ctx, TimedLaunch *tl) {
    if (ctx->timing) ctx->timed.push_back(*tl);
}

int drain_timing(vqm_ctx *ctx) {
    if (ctx->timed.empty()) return 0;
    HIP_TRY(hipStreamSynchronize(ctx->stream));
    for (const TimedLaunch &t : ctx->timed) {
        float ms = 0.f;
        HIP_TRY(hipEventElapsedTime(&ms, t.start, t.stop));
        ctx->time_ms[t.cls] += ms;
        ctx->launches[t.cls] += 1;
        ctx->frames[t.cls] += t.frames;
        ctx->event_pool.push_back(t.start);
        ctx->event_pool.push_back(t.stop);
    }
    ctx->timed.clear();
    return 0;
}

// Launch `launch_expr` (which names the KernelTimer `timer_`), timed when
// the context's timing is on.
#define LAUNCH_TIMED(ctx, cls, frames, launch_expr)                                                \
    do {                                                                                           \
        TimedLaunch tl_;                                                                           \
        vqm::KernelTimer timer_;                                                                   \
        int rc_ = timing_begin(ctx, &tl_, cls, frames, &timer_);                                   \
        if (rc_) return rc_;                                                                       \
        hipError_t e_ = (launch_expr);                                                             \
        if (e_ != hipSuccess) return fail(-EIO, "kernel launch: %s", hipGetErrorString(e_));       \
        timing_end(ctx, &tl_);                                                                     \
    } while (0)

vqm::StepGeometry step_geometry(const Geometry &g) {
    vqm::StepGeometry sg;
    sg.w = g.w;
    sg.h = g.h;
    sg.bpc = g.bpc;
    sg.s = g.s;
    sg.tap = 1.0f / (float)(g.s * g.s);  // formed on the host
    int k = 0;
    while ((1 << k) < g.s) ++k;
    sg.post = ldexpf(1.0f, -(2 * k + g.bpc - 8));
    sg.dec_w = g.dw;
    sg.dec_h = g.dh;
    sg.dec_pitch = g.dpitch;
    sg.packed = vqm::packed_planes(g.s, g.bpc) ? 1 : 0;
    return sg;
}

void fill_map_frame(vqm::SsimFrame &f, const PendingBatch &p, int i, bool decimated) {
    Slot &s = *p.sl[i];
    f.ref = decimated ? static_cast<const void *>(s.planes + s.off_ref[0]) : p.in_r[i];
    f.dis = decimated ? static_cast<const void *>(s.planes + s.off_dis[0]) : p.in_d[i];
    f.partials = s.partials;
    f.result = s.result_dev;
}

// One step launch: decimate `fresh` (may be NULL; at scale 1 it is mapped
// instead, since there is nothing to decimate), map the pipeline's decimated
// batch, finish its mapped batch.  Batches finished by this launch get their
// completion event and leave the pipeline.
int step(vqm_ctx *ctx, PendingBatch *fresh) {
    const Geometry &g = (fresh ? *fresh->sl[0] : *ctx->pipeline.front().sl[0]).geo;
    const bool decimating = g.s > 1;
    vqm::StepRoles r;
    memset(&r, 0, sizeof r);
    PendingBatch *to_map = nullptr, *to_finish = nullptr;
    for (PendingBatch &p : ctx->pipeline) {
        if (p.stage == STAGE_DECIMATED) to_map = &p;
        else if (p.stage == STAGE_MAPPED) to_finish = &p;
    }
    if (fresh && !decimating) to_map = fresh;  // scale 1: mapped straight from the raw planes
    if (fresh && decimating) {
        r.n_dec = fresh->n;
        for (int i = 0; i < fresh->n; ++i) {
            Slot &s = *fresh->sl[i];
            r.dec.f[i].ref = fresh->in_r[i];
            r.dec.f[i].dis = fresh->in_d[i];
            r.dec.f[i].out_ref = s.planes + s.off_ref[0];
            r.dec.f[i].out_dis = s.planes + s.off_dis[0];
        }
    }
    if (to_map) {
        r.n_map = to_map->n;
        for (int i = 0; i < to_map->n; ++i) fill_map_frame(r.map.f[i], *to_map, i, decimating);
    }
    if (to_finish) {
        r.n_fin = to_finish->n;
        for (int i = 0; i < to_finish->n; ++i) {
            fill_map_frame(r.fin.f[i], *to_finish, i, decimating);
            if (to_finish->sl[i]->extra) r.fin_db_mask |= 1u << i;
        }
    }
    const vqm::StepGeometry sg = step_geometry(g);
    // The map reads the decimated planes (uint16 window sums scaled by post,
    // or fp32 values), or the raw samples at scale 1.
    const vqm::InKind kind = decimating ? (sg.packed ? vqm::IN_U16 : vqm::IN_F32)
                                        : (g.bpc == 8 ? vqm::IN_U8 : vqm::IN_U16);
    const int pitch = decimating ? g.dpitch : g.w;
    const float unit = decimating ? (sg.packed ? sg.post : 1.0f) : ldexpf(1.0f, -(g.bpc - 8));
    const int cls = r.n_dec ? VQM_KERNEL_SSIM_STEP : VQM_KERNEL_SSIM_DRAIN;
    LAUNCH_TIMED(ctx, cls, r.n_dec ? r.n_dec : r.n_map,
                 vqm::launch_ssim_step(r, sg, kind, pitch, unit, ctx->taps, ctx->stream, timer_));
    if (to_finish && !ctx->capturing) {
        BatchEvent *be = nullptr;
        int rc = take_batch_event(ctx, &be);
        if (rc) return rc;
        HIP_TRY(hipEventRecord(be->ev, ctx->stream));
        be->refs = to_finish->n;
        be->completed = false;
        for (int i = 0; i < to_finish->n; ++i) to_finish->sl[i]->batch = be;
    }
    // advance the stages (the finished batch is always the oldest)
    if (to_finish) ctx->pipeline.pop_front();
    if (to_map && to_map != fresh) to_map->stage = STAGE_MAPPED;
    if (fresh) {
        fresh->stage = decimating ? STAGE_DECIMATED : STAGE_MAPPED;
        ctx->pipeline.push_back(*fresh);
    }
    return 0;
}

// Run step launches without new work until every pipelined batch is done.
int drain(vqm_ctx *ctx) {
    while (!ctx->pipeline.empty()) {
        int rc = step(ctx, nullptr);
        if (rc) return rc;
    }
    return 0;
}

int enqueue_msssim(vqm_ctx *ctx, Slot *const *sl, int n, const void *const *in_r, const void *const *in_d,
                   hipStream_t stream, bool overlapped = false) {
    const Geometry &g = sl[0]->geo;
    const float unit = ldexpf(1.0f, -(g.bpc - 8));
    for (int j = 0; j < kLevels; ++j) {
        vqm::MsBatch mb;
        memset(&mb, 0, sizeof mb);
        for (int i = 0; i < n; ++i) {
            Slot &s = *sl[i];
            vqm::MsFrame &f = mb.f[i];
            f.ref = j == 0 ? in_r[i] : static_cast<const void *>(s.planes + s.off_ref[j]);
            f.dis = j == 0 ? in_d[i] : static_cast<const void *>(s.planes + s.off_dis[j]);
            f.partials = s.partials + s.span[j];
            f.next_ref = j + 1 < kLevels ? s.planes + s.off_ref[j + 1] : nullptr;
            f.next_dis = j + 1 < kLevels ? s.planes + s.off_dis[j + 1] : nullptr;
        }
        const vqm::InKind kind = j == 0 ? (g.bpc == 8 ? vqm::IN_U8 : vqm::IN_U16) : vqm::IN_F32;
        const int next_pitch = j + 1 < kLevels ? g.lpitch[j + 1] : 0;
        LAUNCH_TIMED(ctx, j == 0 ? VQM_KERNEL_MSSSIM_LEVEL1 : VQM_KERNEL_MSSSIM_COARSE, n,
                     vqm::launch_ms_level(mb, n, kind, g.lpitch[j], g.lw[j], g.lh[j], next_pitch,
                                          j == 0 ? unit : 1.0f, ctx->taps, overlapped, stream, timer_));
    }
    vqm::MsFinishBatch fb;
    memset(&fb, 0, sizeof fb);
    for (int i = 0; i < n; ++i) {
        fb.f[i].partials = sl[i]->partials;
        fb.f[i].result = sl[i]->result_dev;
        if (sl[i]->extra) fb.lcs_mask |= 1u << i;
    }
    vqm::MsLevels lv;
    for (int j = 0; j < kLevels; ++j) {
        lv.nb[j] = vqm::ms_partials(g.lw[j], g.lh[j], n, overlapped);
        lv.offset[j] = (long long)sl[0]->span[j];
        lv.count[j] = (double)(g.lw[j] - 10) * (double)(g.lh[j] - 10);
    }
    const hipError_t e = vqm::launch_ms_finish(fb, n, lv, stream);
    if (e != hipSuccess) return fail(-EIO, "kernel launch: %s", hipGetErrorString(e));
    return 0;
}

// The stream an MS-SSIM batch runs on: every other batch of a caller's
// context on a library-owned stream goes to ms_aux, after the work already
// on the context's stream (its uploads); *overlapped tells the level
// kernels' planner that the batch shares the GPU with the other stream's.
// A caller's stream keeps every batch (the caller orders its own work
// against it), and so do the blocking calls' contexts (each call waits for
// its frame), graph capture and kernel timing (whose events must bracket one
// launch at a time).
int msssim_stream(vqm_ctx *ctx, hipStream_t *out, bool *overlapped) {
    *out = ctx->stream;
    *overlapped = false;
    if (!ctx->ms_overlap || ctx->capturing || ctx->timing) return 0;
    *overlapped = true;
    ctx->ms_flip = !ctx->ms_flip;
    if (!ctx->ms_flip) return 0;
    if (!ctx->ms_aux) {
        HIP_TRY_ALLOC(hipEventCreateWithFlags(&ctx->ms_ready, hipEventDisableTiming));
        HIP_TRY_ALLOC(hipStreamCreate(&ctx->ms_aux));  // blocking, default priority
    }
    HIP_TRY(hipEventRecord(ctx->ms_ready, ctx->stream));
    HIP_TRY(hipStreamWaitEvent(ctx->ms_aux, ctx->ms_ready, 0));
    *out = ctx->ms_aux;
    return 0;
}

int gate(int kind, int w, int h, int bpc) {
    return kind == KIND_SSIM ? gate_ssim(w, h, bpc, nullptr, nullptr, nullptr) : gate_msssim(w, h);
}

// Enqueue n frames of one geometry as one batch: every frame gets the next
// free slot, its own upload, result and completion event; the kernels
// process the whole batch per launch.  `extra`: the finish also writes the
// dB form (float_ssim) or the 15 level means (MS-SSIM) beside the score;
// without it the read-back is the 8-byte score alone.
int submit(vqm_ctx *ctx, int kind, const void *const *refs, const void *const *diss, int n, int w, int h,
           int bpc, bool extra) {
    if (!ctx) return fail(-EINVAL, "NULL context");
    if (!refs || !diss) return fail(-EINVAL, "NULL plane array");
    if (n < 1 || n > VQM_MAX_BATCH) return fail(-EINVAL, "batch of %d frames outside 1..%d", n, VQM_MAX_BATCH);
    for (int i = 0; i < n; ++i) {
        int rc = check_args(refs[i], diss[i], w, h, bpc);
        if (rc) return rc;
    }
    int rc = gate(kind, w, h, bpc);
    if (rc) return rc;
    if (ctx->count + n > VQM_MAX_IN_FLIGHT)
        return fail(-EAGAIN, "%d frames in flight, %d more would exceed %d", ctx->count, n, VQM_MAX_IN_FLIGHT);
    rc = ensure_device(ctx);
    if (rc) return rc;
    const Geometry geo = make_geometry(kind, w, h, bpc);
    // A batch of another geometry or metric first drains the pipeline.
    if (!ctx->pipeline.empty() && !(kind == KIND_SSIM && ctx->pipeline.front().sl[0]->geo == geo)) {
        rc = drain(ctx);
        if (rc) return rc;
    }
    PendingBatch p;
    p.n = n;
    for (int i = 0; i < n; ++i) {
        p.sl[i] = &ctx->slots[(ctx->head + ctx->count + i) % VQM_MAX_IN_FLIGHT];
        rc = prepare_slot(*p.sl[i], geo);
        if (rc) return rc;
        for (int k = 0; k < 16; ++k) p.sl[i]->result_host[k] = NAN;
        p.sl[i]->batch = nullptr;
        p.sl[i]->kind = kind;
        p.sl[i]->extra = extra;
        rc = upload(ctx, *p.sl[i], refs[i], diss[i], &p.in_r[i], &p.in_d[i]);
        if (rc) return rc;
    }
    if (kind == KIND_SSIM) {
        rc = step(ctx, &p);
        if (rc) return rc;
    } else {
        hipStream_t ms = nullptr;
        bool overlapped = false;
        if ((rc = msssim_stream(ctx, &ms, &overlapped))) return rc;
        rc = enqueue_msssim(ctx, p.sl, n, p.in_r, p.in_d, ms, overlapped);
        if (rc) return rc;
        BatchEvent *be = nullptr;
        rc = take_batch_event(ctx, &be);
        if (rc) return rc;
        HIP_TRY(hipEventRecord(be->ev, ms));
        be->refs = n;
        be->completed = false;
        for (int i = 0; i < n; ++i) p.sl[i]->batch = be;
    }
    ctx->count += n;
    return 0;
}

int collect(vqm_ctx *ctx, double *score, double *lcs, double *db) {
    if (!ctx) return fail(-EINVAL, "NULL context");
    if (!score) return fail(-EINVAL, "NULL score pointer");
    if (ctx->count == 0) return fail(-EAGAIN, "no frame in flight");
    int rc = ensure_device(ctx);
    if (rc) return rc;
    Slot &sl = ctx->slots[ctx->head];
    if (sl.batch == nullptr) {
        // Its batch is still in the step pipeline: drain it.
        rc = drain(ctx);
        if (rc) return rc;
    }
    BatchEvent *be = sl.batch;
    if (!be->completed) {
        HIP_TRY(hipEventSynchronize(be->ev));  // the one wait of this frame (and its batch)
        be->completed = true;
    }
    ctx->head = (ctx->head + 1) % VQM_MAX_IN_FLIGHT;
    ctx->count -= 1;
    be->refs -= 1;
    sl.batch = nullptr;
    *score = sl.result_host[0];
    // Without `extra` the finish wrote the score alone; the rest of the block
    // still holds the NaN the submit put there.
    if (lcs && sl.kind == KIND_MSSSIM) memcpy(lcs, sl.result_host + 1, 15 * sizeof(double));
    if (db) *db = sl.kind == KIND_SSIM ? sl.result_host[1] : NAN;
    return 0;
}

// A context on `device`, enqueuing on `stream`, or on a stream of its own
// when `stream` is NULL: a blocking stream (ordered after work on the legacy
// default stream, where torch's default stream enqueues) unless
// `own_nonblocking`.
int create(int device, void *stream, vqm_ctx **out, bool own_nonblocking = false) {
    if (!out) return fail(-EINVAL, "NULL output pointer");
    int n = 0;
    hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess || n == 0) {
        (void)hipGetLastError();
        return fail(-ENODEV, "no HIP device (%s)", hipGetErrorString(e));
    }
    if (device < 0 || device >= n) return fail(-EINVAL, "device %d outside 0..%d", device, n - 1);
    std::unique_ptr<vqm_ctx> ctx(new vqm_ctx());
    ctx->device = device;
    ctx->taps = make_taps();
    int rc = ensure_device(ctx.get());
    if (rc) return rc;
    if (stream) {
        ctx->stream = static_cast<hipStream_t>(stream);
        int sdev = -1;
        if (hipStreamGetDevice(ctx->stream, &sdev) == hipSuccess && sdev != device)
            return fail(-EINVAL, "stream belongs to device %d, context is on %d", sdev, device);
        (void)hipGetLastError();
    } else {
        HIP_TRY(hipStreamCreateWithFlags(&ctx->stream, own_nonblocking ? hipStreamNonBlocking : hipStreamDefault));
        ctx->own_stream = true;
    }
    *out = ctx.release();
    return 0;
}

void destroy(vqm_ctx *ctx) {
    if (!ctx) return;
    int cur = -1;
    (void)hipGetDevice(&cur);
    (void)hipSetDevice(ctx->device);
    (void)hipStreamSynchronize(ctx->stream);
    if (ctx->ms_aux) (void)hipStreamSynchronize(ctx->ms_aux);
    for (Slot &s : ctx->slots) s.release();
    for (auto &be : ctx->batch_events) (void)hipEventDestroy(be->ev);
    for (const TimedLaunch &t : ctx->timed) {
        (void)hipEventDestroy(t.start);
        (void)hipEventDestroy(t.stop);
    }
    for (hipEvent_t e : ctx->event_pool) (void)hipEventDestroy(e);
    if (ctx->ss2_partials) (void)hipFree(ctx->ss2_partials);
    if (ctx->ss2_result_host) (void)hipHostFree(ctx->ss2_result_host);
    ctx->ss2c.release();
    for (Ss2Slot &sl : ctx->ss2_slot) sl.release();
    if (ctx->ms_aux) (void)hipStreamDestroy(ctx->ms_aux);
    if (ctx->ms_ready) (void)hipEventDestroy(ctx->ms_ready);
    if (ctx->own_stream) (void)hipStreamDestroy(ctx->stream);
    if (cur >= 0) (void)hipSetDevice(cur);
    delete ctx;
}

// The blocking calls' contexts: a pool of idle contexts per device.  A
// call leases one (creating it when none is idle), uses it and gives it
// back empty, so the pool holds as many contexts as calls ever ran at once,
// whatever the number of threads that came and went.  Pooled contexts live
// until the process ends: tearing them down at exit could run after the
// HIP runtime itself has been torn down.
std::mutex g_pool_mu;
std::map<int, std::vector<vqm_ctx *>> g_pool;

struct Lease {
    vqm_ctx *ctx = nullptr;
    int dev = 0;
    Lease() = default;
    Lease(const Lease &) = delete;
    Lease &operator=(const Lease &) = delete;
    ~Lease() {
        if (!ctx) return;
        // A context the call left frames in (after an error) goes back only
        // once they are collected; otherwise it is dropped.
        while (ctx->count > 0) {
            double s;
            if (collect(ctx, &s, nullptr, nullptr) != 0) return;
        }
        std::lock_guard<std::mutex> lk(g_pool_mu);
        g_pool[dev].push_back(ctx);
    }
};

int lease_ctx(Lease &l) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(-ENODEV, "no HIP device (%s)", hipGetErrorString(e));
    }
    l.dev = dev;
    {
        std::lock_guard<std::mutex> lk(g_pool_mu);
        std::vector<vqm_ctx *> &idle = g_pool[dev];
        if (!idle.empty()) {
            l.ctx = idle.back();
            idle.pop_back();
            return 0;
        }
    }
    return create(dev, nullptr, &l.ctx);
}

int blocking(int kind, const void *ref, const void *dis, int w, int h, int bpc, double *score, double *lcs,
             double *db) {
    if (!score) return fail(-EINVAL, "NULL score pointer");
    int rc = check_args(ref, dis, w, h, bpc);
    if (rc) return rc;
    rc = gate(kind, w, h, bpc);
    if (rc) return rc;
    Lease lease;
    rc = lease_ctx(lease);
    if (rc) return rc;
    vqm_ctx *ctx = lease.ctx;
    rc = submit(ctx, kind, &ref, &dis, 1, w, h, bpc, lcs != nullptr || db != nullptr);
    if (rc) return rc;
    double s = 0.0, d = 0.0;
    double l[15];
    rc = collect(ctx, &s, l, &d);
    if (rc) return rc;
    *score = s;
    if (lcs) memcpy(lcs, l, sizeof l);
    if (db) *db = d;
    return 0;
}

// Size of one plane of a picture in a chroma layout: Cb and Cr are halved
// horizontally (4:2:0, 4:2:2) and vertically (4:2:0), odd sizes rounding up.
int plane_dims(int w, int h, int chroma, int plane, int *pw, int *ph) {
    if (w <= 0 || h <= 0) return fail(-EINVAL, "size %dx%d", w, h);
    if (chroma < VQM_CHROMA_420 || chroma > VQM_CHROMA_444) return fail(-EINVAL, "unknown chroma layout %d", chroma);
    if (plane < 0 || plane > 2) return fail(-EINVAL, "plane %d outside 0..2", plane);
    const bool sx = plane > 0 && chroma != VQM_CHROMA_444, sy = plane > 0 && chroma == VQM_CHROMA_420;
    if (pw) *pw = sx ? (w + 1) / 2 : w;
    if (ph) *ph = sy ? (h + 1) / 2 : h;
    return 0;
}

// Wait for every frame in flight with one device wait: the stream is in
// order, so once the newest batch has completed every earlier one has too.
int wait_all(vqm_ctx *ctx) {
    if (ctx->count == 0) return 0;
    int rc = drain(ctx);
    if (rc) return rc;
    const Slot &last = ctx->slots[(ctx->head + ctx->count - 1) % VQM_MAX_IN_FLIGHT];
    if (last.batch && !last.batch->completed) {
        HIP_TRY(hipEventSynchronize(last.batch->ev));
        last.batch->completed = true;
    }
    for (int i = 0; i < ctx->count; ++i) {
        Slot &sl = ctx->slots[(ctx->head + i) % VQM_MAX_IN_FLIGHT];
        if (sl.batch) sl.batch->completed = true;
    }
    return 0;
}

// The three planes of a Y'CbCr frame pair: luma as one batch, Cb and Cr (one
// size) as another, one wait, three results.  Every plane is checked and
// gated first, so an error enqueues nothing.
int frame_yuv(int kind, const void *const *ref, const void *const *dis, int w, int h, int bpc, int chroma,
              double *scores, double *lcs, double *db) {
    if (!ref || !dis || !scores) return fail(-EINVAL, "NULL plane array or score pointer");
    int pw[3], ph[3];
    for (int p = 0; p < 3; ++p) {
        int rc = plane_dims(w, h, chroma, p, &pw[p], &ph[p]);
        if (rc) return rc;
        rc = check_args(ref[p], dis[p], pw[p], ph[p], bpc);
        if (rc) return rc;
        rc = gate(kind, pw[p], ph[p], bpc);
        if (rc) return fail(rc, "plane %d (%dx%d): %s", p, pw[p], ph[p], vqm_last_error());
    }
    Lease lease;
    int rc = lease_ctx(lease);
    if (rc) return rc;
    vqm_ctx *ctx = lease.ctx;
    const bool extra = lcs != nullptr || db != nullptr;
    rc = submit(ctx, kind, ref, dis, 1, pw[0], ph[0], bpc, extra);
    if (rc == 0) rc = submit(ctx, kind, ref + 1, dis + 1, 2, pw[1], ph[1], bpc, extra);
    if (rc == 0) rc = wait_all(ctx);
    // Collect whatever was enqueued, so the leased context goes back empty.
    double s[3] = {0.0, 0.0, 0.0}, l[3][15], d[3];
    int n = 0;
    while (ctx->count > 0) {
        const int rc2 = collect(ctx, &s[n < 3 ? n : 2], l[n < 3 ? n : 2], &d[n < 3 ? n : 2]);
        if (rc == 0) rc = rc2;
        if (rc2) break;
        ++n;
    }
    if (rc) return rc;
    for (int p = 0; p < 3; ++p) {
        scores[p] = s[p];
        if (lcs) memcpy(lcs + 15 * p, l[p], sizeof l[p]);
        if (db) db[p] = d[p];
    }
    return 0;
}

// The pipelined scoring loop of vqm_score_frames.
int score_frames(vqm_ctx *const *ctxs, int nctx, int metric, const void *const *refs, const void *const *diss,
                 int n, int w, int h, int bpc, int batch, int lag, double *scores, double *lcs, double *db) {
    if (!ctxs || nctx < 1 || !refs || !diss || !scores) return fail(-EINVAL, "NULL argument or no context");
    if (metric != VQM_METRIC_FLOAT_SSIM && metric != VQM_METRIC_MS_SSIM)
        return fail(-EINVAL, "unknown metric %d", metric);
    if (n < 0) return fail(-EINVAL, "negative frame count");
    if (batch < 1 || batch > VQM_MAX_BATCH) return fail(-EINVAL, "batch %d outside 1..%d", batch, VQM_MAX_BATCH);
    for (int c = 0; c < nctx; ++c) {
        if (!ctxs[c]) return fail(-EINVAL, "NULL context %d", c);
        if (ctxs[c]->count != 0) return fail(-EINVAL, "context %d has frames in flight", c);
    }
    const int kind = metric == VQM_METRIC_MS_SSIM ? KIND_MSSSIM : KIND_SSIM;
    if (lag <= 0) lag = 3 * batch;
    // FIFO of submitted frames: (context, frame index)
    std::vector<std::pair<int, int>> fifo;
    fifo.reserve(n);
    size_t front = 0;
    int rc = 0;
    auto collect_one = [&]() -> int {
        const std::pair<int, int> e = fifo[front++];
        return collect(ctxs[e.first], scores + e.second, lcs ? lcs + 15 * (size_t)e.second : nullptr,
                       db ? db + e.second : nullptr);
    };
    for (int b0 = 0, k = 0; b0 < n && rc == 0; b0 += batch, ++k) {
        const int m = n - b0 < batch ? n - b0 : batch;
        const int c = k % nctx;
        // room in the target context (collecting the oldest frames first)
        while (rc == 0 && front < fifo.size() && ctxs[c]->count + m > VQM_MAX_IN_FLIGHT) rc = collect_one();
        if (rc) break;
        rc = submit(ctxs[c], kind, refs + b0, diss + b0, m, w, h, bpc, lcs != nullptr || db != nullptr);
        if (rc) break;
        for (int i = 0; i < m; ++i) fifo.emplace_back(c, b0 + i);
        // frames with `lag` later frames submitted are due
        const int last = b0 + m - 1;
        while (rc == 0 && front < fifo.size() && fifo[front].second <= last - lag) rc = collect_one();
    }
    while (front < fifo.size()) {
        const int rc2 = collect_one();
        if (rc == 0) rc = rc2;
    }
    return rc;
}

// The statistics' workgroup partials and the one-scale result block.
int ss2_buffers(vqm_ctx *ctx) {
    if (!ctx->ss2_partials) {
        HIP_TRY_ALLOC(hipMalloc(&ctx->ss2_partials, (size_t)vqm::kSs2MaxChannels * vqm::kSs2MaxBlocks * 6 *
                                                        2 * sizeof(float)));
        HIP_TRY_ALLOC(hipHostMalloc(&ctx->ss2_result_host, 6 * vqm::kSs2MaxChannels * sizeof(double),
                                    hipHostMallocMapped | hipHostMallocCoherent));
        HIP_TRY(hipHostGetDevicePointer(reinterpret_cast<void **>(&ctx->ss2_result_dev), ctx->ss2_result_host, 0));
    }
    return 0;
}

// The ssimulacra2 statistics of one scale ("Research-1363: Device-resident
// ssimulacra2 and a single-wait MS-SSIM on SYCL", Finding 4): two launches on
// a leased context's stream, one wait, one read-back of 6 doubles per
// channel.
int ss2_sums(const float *const *planes, int nch, int w, int h, double *sums) {
    if (!planes || !sums) return fail(-EINVAL, "NULL plane array or sums pointer");
    if (nch < 1 || nch > vqm::kSs2MaxChannels)
        return fail(-EINVAL, "%d channels outside 1..%d", nch, vqm::kSs2MaxChannels);
    if (w <= 0 || h <= 0) return fail(-EINVAL, "plane size %dx%d is not positive", w, h);
    if ((long long)w * (long long)h > 0x7fffffffLL) return fail(-EINVAL, "plane %dx%d too large", w, h);
    for (int i = 0; i < 7 * nch; ++i)
        if (!planes[i]) return fail(-EINVAL, "NULL plane %d", i);
    Lease lease;
    int rc = lease_ctx(lease);
    if (rc) return rc;
    vqm_ctx *ctx = lease.ctx;
    for (int i = 0; i < 7 * nch; ++i) {
        PtrKind k;
        rc = classify(planes[i], ctx->device, &k);
        if (rc) return rc;
        if (k != PTR_DEVICE) return fail(-EINVAL, "plane %d: the statistics read device memory only", i);
    }
    rc = ss2_buffers(ctx);
    if (rc) return rc;
    for (int k = 0; k < 6 * nch; ++k) ctx->ss2_result_host[k] = NAN;
    const hipError_t e =
        vqm::launch_ss2_sums(planes, nch, (long long)w * h, ctx->ss2_partials, ctx->ss2_result_dev, ctx->stream);
    if (e != hipSuccess) return fail(-EIO, "kernel launch: %s", hipGetErrorString(e));
    HIP_TRY(hipStreamSynchronize(ctx->stream));  // the one wait
    memcpy(sums, ctx->ss2_result_host, 6 * (size_t)nch * sizeof(double));
    return 0;
}

// ---- the ssimulacra2 per-scale chain ("Research-1363: Device-resident
// ssimulacra2 and a single-wait MS-SSIM on SYCL", Findings 2 and 7)

int check_coef(const float *coef) {
    if (!coef) return fail(-EINVAL, "NULL coefficient array");
    for (int i = 0; i < 4; ++i)
        if (!std::isfinite(coef[i])) return fail(-EINVAL, "coefficient %d is not finite", i);
    return 0;
}

int check_ss2_size(int w, int h) {
    if (w <= 0 || h <= 0) return fail(-EINVAL, "plane size %dx%d is not positive", w, h);
    if ((long long)w * (long long)h > 0x7fffffffLL) return fail(-EINVAL, "plane %dx%d too large", w, h);
    return 0;
}

int device_only(vqm_ctx *ctx, const void *p, const char *what) {
    PtrKind k;
    const int rc = classify(p, ctx->device, &k);
    if (rc) return rc;
    if (k != PTR_DEVICE) return fail(-EINVAL, "%s: the chain reads and writes device memory only", what);
    return 0;
}

// At least `floats` floats of chain workspace and the pinned result block
// (the buffers are idle: a blocking call ends with a wait, a slot is reused
// only after its frame was collected).
int ss2_buffers(Ss2Buffers &b, size_t floats) {
    if (b.work_floats < floats) {
        if (b.work) (void)hipFree(b.work);
        b.work = nullptr;
        b.work_floats = 0;
        HIP_TRY_ALLOC(hipMalloc(&b.work, floats * sizeof(float)));
        b.work_floats = floats;
    }
    if (!b.res_host) {
        HIP_TRY_ALLOC(hipHostMalloc(&b.res_host, 6 * vqm::kSs2MaxChannels * vqm::kSs2MaxScales * sizeof(double),
                                    hipHostMallocMapped | hipHostMallocCoherent));
        HIP_TRY(hipHostGetDevicePointer(reinterpret_cast<void **>(&b.res_dev), b.res_host, 0));
    }
    return 0;
}

// One plane through the row pass and the column pass.
int ss2_blur_plane(const float *in, float *out, int w, int h, const float *coef) {
    if (!in || !out) return fail(-EINVAL, "NULL plane pointer");
    int rc = check_ss2_size(w, h);
    if (!rc) rc = check_coef(coef);
    if (rc) return rc;
    Lease lease;
    rc = lease_ctx(lease);
    if (rc) return rc;
    vqm_ctx *ctx = lease.ctx;
    if ((rc = device_only(ctx, in, "input plane")) || (rc = device_only(ctx, out, "output plane"))) return rc;
    if ((rc = ss2_buffers(ctx->ss2c, vqm::ss2_chain_scratch_floats(1, 1, &w, &h, 1)))) return rc;
    vqm::Ss2ChainArgs args{};
    vqm::Ss2Scale &sc = args.scale[0];
    sc.w = w;
    sc.h = h;
    sc.pstride = (long long)w * h;
    sc.a[0] = in;
    sc.rows[0] = out;  // the row pass writes out, the column pass then works in place
    sc.out[0] = out;
    args.nscales = 1;
    args.nch = 1;
    args.nplanes = 1;
    args.stats = false;
    memcpy(args.coef, coef, sizeof args.coef);
    args.scratch = ctx->ss2c.work;
    const vqm::KernelTimer none;
    const hipError_t e = vqm::launch_ss2_chain(args, ctx->stream, none, none);
    if (e != hipSuccess) return fail(-EIO, "kernel launch: %s", hipGetErrorString(e));
    HIP_TRY(hipStreamSynchronize(ctx->stream));
    return 0;
}

int ss2_down_plane(const float *in, float *out, int w, int h) {
    if (!in || !out) return fail(-EINVAL, "NULL plane pointer");
    int rc = check_ss2_size(w, h);
    if (rc) return rc;
    Lease lease;
    rc = lease_ctx(lease);
    if (rc) return rc;
    vqm_ctx *ctx = lease.ctx;
    if ((rc = device_only(ctx, in, "input plane")) || (rc = device_only(ctx, out, "output plane"))) return rc;
    const hipError_t e = vqm::launch_ss2_pyramid(&in, &out, 1, w, h, 1, ctx->stream);
    if (e != hipSuccess) return fail(-EIO, "kernel launch: %s", hipGetErrorString(e));
    HIP_TRY(hipStreamSynchronize(ctx->stream));
    return 0;
}

using vqm::kSs2MaxScales;

size_t align64(size_t n) { return (n + 63) & ~(size_t)63; }

// The arguments of one frame of the chain, checked on the host before any
// HIP call.
int ss2_check(const float *const *ref, const float *const *dis, int nch, int w, int h, int nscales,
              const float *coef) {
    if (!ref || !dis) return fail(-EINVAL, "NULL plane array");
    if (nch < 1 || nch > vqm::kSs2MaxChannels)
        return fail(-EINVAL, "%d channels outside 1..%d", nch, vqm::kSs2MaxChannels);
    if (nscales < 1 || nscales > kSs2MaxScales)
        return fail(-EINVAL, "%d scales outside 1..%d", nscales, kSs2MaxScales);
    int rc = check_ss2_size(w, h);
    if (!rc) rc = check_coef(coef);
    if (rc) return rc;
    for (int c = 0; c < nch; ++c)
        if (!ref[c] || !dis[c]) return fail(-EINVAL, "NULL plane of channel %d", c);
    return 0;
}

// Every scale of one frame enqueued on `stream`: the pyramid of the two
// pictures (one launch for every later scale), then the row pass of every
// scale with the products, the column pass of every scale with the
// statistics, and the sums of each (scale, channel)'s partials into buf's
// pinned result block (6 * nch * nscales doubles, NaN until written).
//
// blurred (inspection only): per channel a device buffer that also receives
// the blurred planes mu1, mu2, s11, s22, s12 from the same kernels, the five
// planes of each scale (tightly packed) after those of the scales before it.
int ss2_enqueue(hipStream_t stream, Ss2Buffers &buf, const float *const *ref, const float *const *dis, int nch,
                int w, int h, int nscales, const float *coef, float *const *blurred = nullptr) {
    int rc = 0;
    // The workspace: the chain's checkpoints and partials, then per scale
    // the five row-blurred planes of every channel, then the two images of
    // every channel of every later scale.
    int sw[kSs2MaxScales], sh[kSs2MaxScales];
    size_t ps[kSs2MaxScales], rows_off[kSs2MaxScales], pyr_off[kSs2MaxScales] = {0};
    sw[0] = w;
    sh[0] = h;
    for (int s = 1; s < nscales; ++s) vqm::ss2_downsampled_dim(sw[s - 1], sh[s - 1], &sw[s], &sh[s]);
    size_t total = align64(vqm::ss2_chain_scratch_floats(nch, 5, sw, sh, nscales));
    for (int s = 0; s < nscales; ++s) {
        ps[s] = blurred ? (size_t)sw[s] * sh[s] : align64((size_t)sw[s] * sh[s]);
        rows_off[s] = total;
        total += 5 * (size_t)nch * ps[s];
    }
    for (int s = 1; s < nscales; ++s) {
        pyr_off[s] = total;
        total += 2 * (size_t)nch * ps[s];
    }
    if ((rc = ss2_buffers(buf, total))) return rc;
    const int nres = 6 * nch * nscales;
    for (int k = 0; k < nres; ++k) buf.res_host[k] = NAN;

    float *const work = buf.work;
    vqm::Ss2ChainArgs args{};
    args.nscales = nscales;
    args.nch = nch;
    args.nplanes = 5;
    args.stats = true;
    memcpy(args.coef, coef, sizeof args.coef);
    args.scratch = work;
    args.result = buf.res_dev;
    // images: the caller's at the first scale, the pyramid's after it
    // (plane 2c the reference, 2c + 1 the distorted one; pyr holds scale
    // s's plane i at (s - 1) * 2 nch + i)
    const float *img[2 * vqm::kSs2MaxChannels];
    float *pyr[(kSs2MaxScales - 1) * 2 * vqm::kSs2MaxChannels];
    size_t blurred_off = 0;  // floats of the earlier scales' blurred planes
    for (int s = 0; s < nscales; ++s) {
        vqm::Ss2Scale &sc = args.scale[s];
        sc.w = sw[s];
        sc.h = sh[s];
        sc.pstride = (long long)ps[s];
        for (int c = 0; c < nch; ++c) {
            sc.rows[c] = work + rows_off[s] + 5 * (size_t)c * ps[s];
            sc.out[c] = blurred ? blurred[c] + blurred_off : nullptr;
            if (s == 0) {
                sc.a[c] = img[2 * c] = ref[c];
                sc.b[c] = img[2 * c + 1] = dis[c];
                continue;
            }
            float *const a = work + pyr_off[s] + (2 * (size_t)c) * ps[s], *const b = a + ps[s];
            pyr[(s - 1) * 2 * nch + 2 * c] = a;
            pyr[(s - 1) * 2 * nch + 2 * c + 1] = b;
            sc.a[c] = a;
            sc.b[c] = b;
        }
        blurred_off += 5 * (size_t)sw[s] * sh[s];
    }
    hipError_t e = hipSuccess;
    if (nscales > 1) e = vqm::launch_ss2_pyramid(img, pyr, 2 * nch, w, h, nscales - 1, stream);
    const vqm::KernelTimer none;
    if (e == hipSuccess) e = vqm::launch_ss2_chain(args, stream, none, none);
    if (e != hipSuccess) return fail(-EIO, "kernel launch: %s", hipGetErrorString(e));
    return 0;
}

// Every plane of a chain frame on the context's device.
int ss2_device_planes(vqm_ctx *ctx, const float *const *ref, const float *const *dis, int nch,
                      float *const *blurred = nullptr) {
    int rc = 0;
    for (int c = 0; c < nch; ++c)
        if ((rc = device_only(ctx, ref[c], "reference plane")) || (rc = device_only(ctx, dis[c], "distorted plane")) ||
            (blurred && (rc = device_only(ctx, blurred[c], "blurred planes"))))
            return rc;
    return 0;
}

// A frame's chain as one blocking call on a leased context: enqueue, one
// wait, one read-back.
int ss2_chain(const float *const *ref, const float *const *dis, int nch, int w, int h, int nscales,
              const float *coef, double *sums, float *const *blurred = nullptr) {
    if (!sums) return fail(-EINVAL, "NULL sums pointer");
    int rc = ss2_check(ref, dis, nch, w, h, nscales, coef);
    if (rc) return rc;
    Lease lease;
    rc = lease_ctx(lease);
    if (rc) return rc;
    vqm_ctx *ctx = lease.ctx;
    if ((rc = ss2_device_planes(ctx, ref, dis, nch, blurred))) return rc;
    rc = ss2_enqueue(ctx->stream, ctx->ss2c, ref, dis, nch, w, h, nscales, coef, blurred);
    if (rc) return rc;
    HIP_TRY(hipStreamSynchronize(ctx->stream));  // the one wait
    memcpy(sums, ctx->ss2c.res_host, 6 * (size_t)nch * nscales * sizeof(double));
    return 0;
}

// Submit: the frame goes to the next free slot, on the slot's own stream,
// after the work already on the context's stream; no wait.
int ss2_submit(vqm_ctx *ctx, const float *const *ref, const float *const *dis, int nch, int w, int h,
               int nscales, const float *coef) {
    if (!ctx) return fail(-EINVAL, "NULL context");
    int rc = ss2_check(ref, dis, nch, w, h, nscales, coef);
    if (rc) return rc;
    if (ctx->ss2_count >= VQM_SS2_MAX_IN_FLIGHT)
        return fail(-EAGAIN, "%d ssimulacra2 frames already in flight", ctx->ss2_count);
    if ((rc = ensure_device(ctx)) || (rc = ss2_device_planes(ctx, ref, dis, nch))) return rc;
    Ss2Slot &sl = ctx->ss2_slot[(ctx->ss2_head + ctx->ss2_count) % VQM_SS2_MAX_IN_FLIGHT];
    if (!sl.stream) {
        HIP_TRY_ALLOC(hipStreamCreate(&sl.stream));  // a blocking stream, default priority
        HIP_TRY_ALLOC(hipEventCreateWithFlags(&sl.ready, hipEventDisableTiming));
        HIP_TRY_ALLOC(hipEventCreateWithFlags(&sl.done, hipEventDisableTiming));
    }
    HIP_TRY(hipEventRecord(sl.ready, ctx->stream));
    HIP_TRY(hipStreamWaitEvent(sl.stream, sl.ready, 0));
    rc = ss2_enqueue(sl.stream, sl.buf, ref, dis, nch, w, h, nscales, coef);
    if (rc) return rc;
    HIP_TRY(hipEventRecord(sl.done, sl.stream));
    sl.nres = 6 * nch * nscales;
    ++ctx->ss2_count;
    return 0;
}

// Collect: the oldest submitted frame's one wait and read-back.
int ss2_collect(vqm_ctx *ctx, double *sums) {
    if (!ctx || !sums) return fail(-EINVAL, "NULL context or sums pointer");
    if (ctx->ss2_count == 0) return fail(-EAGAIN, "no ssimulacra2 frame in flight");
    int rc = ensure_device(ctx);
    if (rc) return rc;
    Ss2Slot &sl = ctx->ss2_slot[ctx->ss2_head];
    HIP_TRY(hipEventSynchronize(sl.done));  // the one wait
    memcpy(sums, sl.buf.res_host, (size_t)sl.nres * sizeof(double));
    ctx->ss2_head = (ctx->ss2_head + 1) % VQM_SS2_MAX_IN_FLIGHT;
    --ctx->ss2_count;
    return 0;
}

// Three symmetric exponential smoothers in series with variance sigma^2.
int ss2_cascade(double sigma, float *coef) {
    if (!coef) return fail(-EINVAL, "NULL coefficient array");
    if (!(sigma > 0.0) || !(sigma < 1e6)) return fail(-EINVAL, "sigma %g outside (0, 1e6)", sigma);
    // one smoother with pole p has variance 2p / (1 - p)^2; three have
    // 6p / (1 - p)^2.  p is the smaller root of
    // sigma^2 p^2 - (2 sigma^2 + 6) p + sigma^2 = 0, the one in (0, 1).
    const double v = sigma * sigma;
    const double p = ((v + 3.0) - std::sqrt(6.0 * v + 9.0)) / v;
    const double g = 1.0 - p;
    coef[0] = (float)(g * g * g);
    coef[1] = (float)(3.0 * p);
    coef[2] = (float)(-3.0 * p * p);
    coef[3] = (float)(p * p * p);
    return 0;
}

// The read-ceiling probe: `reps` timed launches of the streaming read over a
// device buffer, on a leased context's stream; the mean kernel time.
int read_probe(const void *buf, long long bytes, int reps, double *ms) {
    if (!buf || !ms) return fail(-EINVAL, "NULL argument");
    if (bytes < 16 || reps < 1) return fail(-EINVAL, "need at least 16 bytes and one repetition");
    Lease lease;
    int rc = lease_ctx(lease);
    if (rc) return rc;
    vqm_ctx *ctx = lease.ctx;
    PtrKind k;
    rc = classify(buf, ctx->device, &k);
    if (rc) return rc;
    if (k != PTR_DEVICE) return fail(-EINVAL, "the probe reads device memory only");
    const long long blocks = vqm::read_probe_blocks(bytes);
    if (blocks > 0x7fffffffLL) return fail(-EINVAL, "%lld bytes are too many for one probe launch", bytes);
    uint32_t *sink = nullptr;
    HIP_TRY_ALLOC(hipMalloc(&sink, (size_t)blocks * sizeof(uint32_t)));
    hipEvent_t ev[2] = {nullptr, nullptr};
    hipError_t e = hipEventCreate(&ev[0]);
    if (e == hipSuccess) e = hipEventCreate(&ev[1]);
    double total = 0.0;
    for (int r = 0; r <= reps && e == hipSuccess; ++r) {  // launch 0 warms up
        vqm::KernelTimer kt;
        kt.start = ev[0];
        kt.stop = ev[1];
        e = vqm::launch_read_probe(buf, bytes, sink, ctx->stream, kt);
        if (e == hipSuccess) e = hipEventSynchronize(ev[1]);
        float t = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&t, ev[0], ev[1]);
        if (r > 0) total += t;
    }
    for (hipEvent_t x : ev)
        if (x) (void)hipEventDestroy(x);
    (void)hipFree(sink);
    if (e != hipSuccess) return fail(-EIO, "read probe: %s", hipGetErrorString(e));
    *ms = total / reps;
    return 0;
}

int valu_probe(int waves_per_simd, int iters, int reps, double *tflops) {
    if (!tflops) return fail(-EINVAL, "NULL argument");
    if (waves_per_simd < 1 || waves_per_simd > 32 || iters < 1 || iters > (1 << 20) || reps < 1)
        return fail(-EINVAL, "waves per SIMD 1..32, iterations 1..2^20 and one repetition at least");
    Lease lease;
    int rc = lease_ctx(lease);
    if (rc) return rc;
    vqm_ctx *ctx = lease.ctx;
    hipDeviceProp_t prop;
    HIP_TRY(hipGetDeviceProperties(&prop, ctx->device));
    // four waves of 64 per workgroup, four SIMDs per compute unit
    const int blocks = waves_per_simd * prop.multiProcessorCount;
    float *out = nullptr;
    HIP_TRY_ALLOC(hipMalloc(&out, (size_t)blocks * 256 * sizeof(float)));
    hipEvent_t ev[2] = {nullptr, nullptr};
    hipError_t e = hipEventCreate(&ev[0]);
    if (e == hipSuccess) e = hipEventCreate(&ev[1]);
    double total = 0.0;
    for (int r = 0; r <= reps && e == hipSuccess; ++r) {  // launch 0 warms up
        vqm::KernelTimer kt;
        kt.start = ev[0];
        kt.stop = ev[1];
        e = vqm::launch_valu_probe(out, blocks, iters, ctx->stream, kt);
        if (e == hipSuccess) e = hipEventSynchronize(ev[1]);
        float t = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&t, ev[0], ev[1]);
        if (r > 0) total += t;
    }
    for (hipEvent_t x : ev)
        if (x) (void)hipEventDestroy(x);
    (void)hipFree(out);
    if (e != hipSuccess) return fail(-EIO, "VALU probe: %s", hipGetErrorString(e));
    const double ms = total / reps;
    *tflops = 2.0 * (double)vqm::valu_probe_fmas(blocks, iters) / (ms * 1e-3) / 1e12;
    return 0;
}

int pair_ops(int op, const float *a, const float *b, float *out, int n) {
    if (!a || !b || !out) return fail(-EINVAL, "NULL argument");
    if (op < 0 || op > 4) return fail(-EINVAL, "pair operation %d outside 0..4", op);
    if (n < 1 || n > (1 << 24)) return fail(-EINVAL, "%d elements outside 1..2^24", n);
    Lease lease;
    int rc = lease_ctx(lease);
    if (rc) return rc;
    vqm_ctx *ctx = lease.ctx;
    const size_t bytes = 2 * (size_t)n * sizeof(float);
    float *d = nullptr;
    HIP_TRY_ALLOC(hipMalloc(&d, 3 * bytes));
    float *da = d, *db = d + 2 * (size_t)n, *dout = d + 4 * (size_t)n;
    hipError_t e = hipMemcpyAsync(da, a, bytes, hipMemcpyHostToDevice, ctx->stream);
    if (e == hipSuccess) e = hipMemcpyAsync(db, b, bytes, hipMemcpyHostToDevice, ctx->stream);
    if (e == hipSuccess) e = vqm::launch_pair_ops(op, da, db, dout, n, ctx->stream);
    if (e == hipSuccess) e = hipMemcpyAsync(out, dout, bytes, hipMemcpyDeviceToHost, ctx->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(ctx->stream);
    (void)hipFree(d);
    if (e != hipSuccess) return fail(-EIO, "pair operations: %s", hipGetErrorString(e));
    return 0;
}

// One frame into the next free slot for the debug exports (synchronous; the
// slot is not counted as in flight).
int debug_slot(vqm_ctx *ctx, const Geometry &g, const void *ref, const void *dis, Slot **sl_out,
               const void **dref, const void **ddis) {
    if (ctx->count >= VQM_MAX_IN_FLIGHT) return fail(-EAGAIN, "%d frames already in flight", ctx->count);
    int rc = ensure_device(ctx);
    if (rc) return rc;
    Slot &sl = ctx->slots[(ctx->head + ctx->count) % VQM_MAX_IN_FLIGHT];
    rc = prepare_slot(sl, g);
    if (rc) return rc;
    rc = upload(ctx, sl, ref, dis, dref, ddis);
    if (rc) return rc;
    *sl_out = &sl;
    return 0;
}

}  // namespace

// A recorded scoring pass over a fixed set of device-resident frames
// ("ADR-1357: Run the SYCL CAMBI extractor entirely on the device", Decision
// and Consequences: the kernels register once with a combined graph and its
// replay absorbs their launches; "Research-1363: Device-resident ssimulacra2
// and a single-wait MS-SSIM on SYCL", Finding 6: one wait per pass).  It owns
// a private context, whose first n slots hold the frames' scratch and
// results for the graph's lifetime.
struct vqm_graph {
    vqm_ctx *ctx = nullptr;
    int kind = KIND_NONE;
    int n = 0;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    hipEvent_t done = nullptr;
    bool pending = false;  // launched and not yet collected
};

namespace {

// Record every launch of one pass over the frames (float_ssim: the step
// pipeline and its drain; MS-SSIM: five levels and the combine per batch)
// into g->graph.  The frames are device memory, so the pass has no copies;
// it records no events and no memsets.
int record_pass(vqm_graph *g, const void *const *refs, const void *const *dis, int w, int h, int bpc,
                int batch) {
    vqm_ctx *ctx = g->ctx;
    const Geometry geo = make_geometry(g->kind, w, h, bpc);
    for (int i = 0; i < g->n; ++i) {
        int rc = prepare_slot(ctx->slots[i], geo);
        if (rc) return rc;
        for (int k = 0; k < 16; ++k) ctx->slots[i].result_host[k] = NAN;
        ctx->slots[i].extra = true;  // a replay's collect may ask for every output
    }
    HIP_TRY(hipStreamBeginCapture(ctx->stream, hipStreamCaptureModeThreadLocal));
    ctx->capturing = true;
    int rc = 0;
    for (int b0 = 0; b0 < g->n && rc == 0; b0 += batch) {
        PendingBatch p;
        p.n = g->n - b0 < batch ? g->n - b0 : batch;
        for (int i = 0; i < p.n; ++i) {
            p.sl[i] = &ctx->slots[b0 + i];
            p.in_r[i] = refs[b0 + i];
            p.in_d[i] = dis[b0 + i];
        }
        rc = g->kind == KIND_SSIM ? step(ctx, &p) : enqueue_msssim(ctx, p.sl, p.n, p.in_r, p.in_d, ctx->stream);
    }
    if (rc == 0 && g->kind == KIND_SSIM) rc = drain(ctx);
    ctx->capturing = false;
    ctx->pipeline.clear();
    hipGraph_t graph = nullptr;
    const hipError_t e = hipStreamEndCapture(ctx->stream, &graph);
    if (rc) {
        if (graph) (void)hipGraphDestroy(graph);
        return rc;
    }
    if (e != hipSuccess) return fail(-EIO, "hipStreamEndCapture: %s", hipGetErrorString(e));
    g->graph = graph;
    HIP_TRY(hipGraphInstantiateWithFlags(&g->exec, g->graph, 0));
    return 0;
}

void destroy_graph(vqm_graph *g) {
    if (!g) return;
    if (g->ctx) {
        int cur = -1;
        (void)hipGetDevice(&cur);
        (void)hipSetDevice(g->ctx->device);
        (void)hipStreamSynchronize(g->ctx->stream);
        if (g->exec) (void)hipGraphExecDestroy(g->exec);
        if (g->graph) (void)hipGraphDestroy(g->graph);
        if (g->done) (void)hipEventDestroy(g->done);
        if (cur >= 0) (void)hipSetDevice(cur);
        destroy(g->ctx);
    }
    delete g;
}

int graph_create(int device, void *stream, int metric, const void *const *refs, const void *const *dis, int n,
                 int w, int h, int bpc, int batch, vqm_graph **out) {
    if (!out) return fail(-EINVAL, "NULL output pointer");
    *out = nullptr;
    if (metric != VQM_METRIC_FLOAT_SSIM && metric != VQM_METRIC_MS_SSIM)
        return fail(-EINVAL, "unknown metric %d", metric);
    if (!refs || !dis) return fail(-EINVAL, "NULL plane array");
    if (n < 1 || n > VQM_MAX_IN_FLIGHT) return fail(-EINVAL, "%d frames outside 1..%d", n, VQM_MAX_IN_FLIGHT);
    if (batch < 1 || batch > VQM_MAX_BATCH) return fail(-EINVAL, "batch %d outside 1..%d", batch, VQM_MAX_BATCH);
    for (int i = 0; i < n; ++i) {
        int rc = check_args(refs[i], dis[i], w, h, bpc);
        if (rc) return rc;
    }
    const int kind = metric == VQM_METRIC_MS_SSIM ? KIND_MSSSIM : KIND_SSIM;
    int rc = gate(kind, w, h, bpc);
    if (rc) return rc;
    std::unique_ptr<vqm_graph, void (*)(vqm_graph *)> g(new vqm_graph(), destroy_graph);
    g->kind = kind;
    g->n = n;
    rc = create(device, stream, &g->ctx, /*own_nonblocking=*/true);
    if (rc) return rc;
    for (int i = 0; i < n; ++i)
        for (const void *p : {refs[i], dis[i]}) {
            PtrKind k;
            rc = classify(p, device, &k);
            if (rc) return rc;
            if (k != PTR_DEVICE) return fail(-EINVAL, "frame %d: a recorded pass takes device memory only", i);
        }
    HIP_TRY(hipEventCreateWithFlags(&g->done, kResultEventFlags));
    rc = record_pass(g.get(), refs, dis, w, h, bpc, batch);
    if (rc) return rc;
    *out = g.release();
    return 0;
}

int graph_launch(vqm_graph *g) {
    if (!g) return fail(-EINVAL, "NULL graph");
    if (g->pending) return fail(-EBUSY, "the previous replay has not been collected");
    int rc = ensure_device(g->ctx);
    if (rc) return rc;
    HIP_TRY(hipGraphLaunch(g->exec, g->ctx->stream));
    HIP_TRY(hipEventRecord(g->done, g->ctx->stream));
    g->pending = true;
    return 0;
}

int graph_collect(vqm_graph *g, double *scores, double *lcs, double *db) {
    if (!g || !scores) return fail(-EINVAL, "NULL argument");
    if (!g->pending) return fail(-EAGAIN, "no replay in flight");
    int rc = ensure_device(g->ctx);
    if (rc) return rc;
    HIP_TRY(hipEventSynchronize(g->done));  // the one wait of the replay
    g->pending = false;
    for (int i = 0; i < g->n; ++i) {
        const Slot &sl = g->ctx->slots[i];
        scores[i] = sl.result_host[0];
        if (lcs && g->kind == KIND_MSSSIM) memcpy(lcs + 15 * (size_t)i, sl.result_host + 1, 15 * sizeof(double));
        if (db) db[i] = g->kind == KIND_SSIM ? sl.result_host[1] : NAN;
    }
    return 0;
}

// ---- the allocation-free float_ssim pass (vqm_ssim_frame_noalloc) ----
//
// Its scratch (both decimated planes and the map's partial sums) lives in one
// file-scope device array per GPU, which each GPU the library runs on holds
// until the process ends.  In host code the array's name only stands in for
// the symbol: its device address comes from hipGetSymbolAddress, taken once
// per device with that device current, and only that address ever reaches a
// kernel.  Every call on a device shares the array, so calls that overlap on
// one GPU race; the kernels overwrite every byte they later read, so nothing
// needs clearing between calls.
static __device__ __align__(256) unsigned char scratch[VQM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxScratchDevices] = {};

int noalloc_scratch(int device, unsigned char **out) {
    if (device < 0 || device >= kMaxScratchDevices)
        return fail(-EINVAL, "device %d outside the 0..%d the allocation-free path serves", device,
                    kMaxScratchDevices - 1);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_dev[device]) {
        void *ptr = nullptr;
        HIP_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));  // the current device is `device`
        if (!ptr) return fail(-EIO, "hipGetSymbolAddress returned no address for the scratch array");
        g_scratch_dev[device] = ptr;
    }
    *out = static_cast<unsigned char *>(g_scratch_dev[device]);
    return 0;
}

// Device-visible address of the caller's score buffer: device memory of
// `device`, or pinned host memory (its mapped address).
int noalloc_result(double *score, int device, double **dev) {
    hipPointerAttribute_t a;
    memset(&a, 0, sizeof a);
    if (hipPointerGetAttributes(&a, score) != hipSuccess) {
        (void)hipGetLastError();
        return fail(-EINVAL, "score must be device memory or pinned host memory");
    }
    if (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged) {
        if (a.device != device)
            return fail(-EINVAL, "score is device memory of device %d, the call runs on %d", a.device, device);
        *dev = score;
        return 0;
    }
    if (a.type == hipMemoryTypeHost && a.devicePointer) {
        *dev = static_cast<double *>(a.devicePointer);
        return 0;
    }
    return fail(-EINVAL, "score must be device memory or pinned host memory");
}

int ssim_noalloc(const void *ref, const void *dis, int w, int h, int bpc, double *score, void *stream) {
    if (!score) return fail(-EINVAL, "NULL score pointer");
    int rc = check_args(ref, dis, w, h, bpc);
    if (rc) return rc;
    rc = gate_ssim(w, h, bpc, nullptr, nullptr, nullptr);
    if (rc) return rc;
    const Geometry g = make_geometry(KIND_SSIM, w, h, bpc);
    // Scratch: two decimated planes (none at scale 1: the map reads the raw
    // samples), then one double per map tile.
    const size_t plane_bytes = g.s > 1 ? (size_t)g.dpitch * (size_t)g.dh * sizeof(float) : 0;
    const size_t planes_bytes = (2 * plane_bytes + 255) / 256 * 256;
    const size_t need = planes_bytes + (size_t)vqm::ssim_partials(g.dw, g.dh) * sizeof(double);
    if (need > (size_t)VQM_NOALLOC_SCRATCH_BYTES)
        return fail(-ENOSPC, "a %dx%d frame needs %zu bytes of scratch; the allocation-free path holds %d", w, h,
                    need, VQM_NOALLOC_SCRATCH_BYTES);
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (st) {
        int sdev = -1;
        if (hipStreamGetDevice(st, &sdev) == hipSuccess && sdev != dev)
            return fail(-EINVAL, "stream belongs to device %d, the current device is %d", sdev, dev);
        (void)hipGetLastError();
    }
    for (const void *p : {ref, dis}) {
        PtrKind k;
        rc = classify(p, dev, &k);
        if (rc) return rc;
        if (k != PTR_DEVICE) return fail(-EINVAL, "the allocation-free path reads device planes only");
    }
    double *result = nullptr;
    rc = noalloc_result(score, dev, &result);
    if (rc) return rc;
    unsigned char *base = nullptr;
    rc = noalloc_scratch(dev, &base);
    if (rc) return rc;

    static const vqm::Taps taps = make_taps();
    const vqm::StepGeometry sg = step_geometry(g);
    const bool decimating = g.s > 1;
    void *out_ref = base, *out_dis = base + plane_bytes;
    double *partials = reinterpret_cast<double *>(base + planes_bytes);
    const vqm::KernelTimer no_timer;
    vqm::StepRoles r;
    // The same step kernel as the pipelined path, one role per launch:
    // decimate, map, finish (no decimation at scale 1).
    if (decimating) {
        memset(&r, 0, sizeof r);
        r.n_dec = 1;
        r.dec.f[0] = vqm::DecimateFrame{ref, dis, out_ref, out_dis};
        const hipError_t e = vqm::launch_ssim_step(r, sg, sg.packed ? vqm::IN_U16 : vqm::IN_F32, g.dpitch,
                                                   sg.packed ? sg.post : 1.0f, taps, st, no_timer);
        if (e != hipSuccess) return fail(-EIO, "kernel launch: %s", hipGetErrorString(e));
    }
    const vqm::InKind kind = decimating ? (sg.packed ? vqm::IN_U16 : vqm::IN_F32)
                                        : (g.bpc == 8 ? vqm::IN_U8 : vqm::IN_U16);
    const int pitch = decimating ? g.dpitch : g.w;
    const float unit = decimating ? (sg.packed ? sg.post : 1.0f) : ldexpf(1.0f, -(g.bpc - 8));
    const vqm::SsimFrame f{decimating ? out_ref : ref, decimating ? out_dis : dis, partials, result};
    for (int role = 0; role < 2; ++role) {
        memset(&r, 0, sizeof r);
        if (role == 0) {
            r.n_map = 1;
            r.map.f[0] = f;
        } else {
            r.n_fin = 1;
            r.fin.f[0] = f;
        }
        const hipError_t e = vqm::launch_ssim_step(r, sg, kind, pitch, unit, taps, st, no_timer);
        if (e != hipSuccess) return fail(-EIO, "kernel launch: %s", hipGetErrorString(e));
    }
    return 0;
}

}  // namespace

extern "C" {

int vqm_abi_version(void) { return VQM_ABI_VERSION; }

int vqm_ssim_frame_noalloc(const void *ref, const void *dis, int w, int h, int bpc, double *score,
                           void *hip_stream) {
    return ssim_noalloc(ref, dis, w, h, bpc, score, hip_stream);
}

int vqm_graph_create(int device, void *hip_stream, int metric, const void *const *refs, const void *const *dis,
                     int n, int w, int h, int bpc, int batch, vqm_graph **out) {
    DeviceScope scope;
    return graph_create(device, hip_stream, metric, refs, dis, n, w, h, bpc, batch, out);
}

int vqm_graph_launch(vqm_graph *g) {
    DeviceScope scope;
    return graph_launch(g);
}

int vqm_graph_collect(vqm_graph *g, double *scores, double *lcs, double *db) {
    DeviceScope scope;
    return graph_collect(g, scores, lcs, db);
}

void vqm_graph_destroy(vqm_graph *g) { destroy_graph(g); }

int vqm_ssim_scale(int w, int h) {
    if (w <= 0 || h <= 0) return 0;
    return scale_of(w, h);
}

int vqm_ssim_geometry(int w, int h, int bpc, int *scale, int *dec_w, int *dec_h) {
    return gate_ssim(w, h, bpc, scale, dec_w, dec_h);
}

int vqm_ssim_frame(const void *ref, const void *dis, int w, int h, int bpc, double *score) {
    return blocking(KIND_SSIM, ref, dis, w, h, bpc, score, nullptr, nullptr);
}

int vqm_ssim_frame_db(const void *ref, const void *dis, int w, int h, int bpc, double *score, double *db) {
    if (!db) return fail(-EINVAL, "NULL db pointer");
    return blocking(KIND_SSIM, ref, dis, w, h, bpc, score, nullptr, db);
}

int vqm_msssim_frame(const void *ref, const void *dis, int w, int h, int bpc, double *score) {
    return blocking(KIND_MSSSIM, ref, dis, w, h, bpc, score, nullptr, nullptr);
}

int vqm_msssim_frame_lcs(const void *ref, const void *dis, int w, int h, int bpc, double *score,
                         double *lcs) {
    if (!lcs) return fail(-EINVAL, "NULL lcs pointer");
    return blocking(KIND_MSSSIM, ref, dis, w, h, bpc, score, lcs, nullptr);
}

int vqm_plane_dims(int w, int h, int chroma, int plane, int *pw, int *ph) {
    return plane_dims(w, h, chroma, plane, pw, ph);
}

int vqm_ssim_frame_yuv(const void *const *ref, const void *const *dis, int w, int h, int bpc, int chroma,
                       double *scores, double *db) {
    return frame_yuv(KIND_SSIM, ref, dis, w, h, bpc, chroma, scores, nullptr, db);
}

int vqm_msssim_frame_yuv(const void *const *ref, const void *const *dis, int w, int h, int bpc, int chroma,
                         double *scores, double *lcs) {
    return frame_yuv(KIND_MSSSIM, ref, dis, w, h, bpc, chroma, scores, lcs, nullptr);
}

int vqm_ctx_create(int device, void *hip_stream, vqm_ctx **out) {
    DeviceScope scope;
    const int rc = create(device, hip_stream, out);
    // The blocking calls' pooled contexts wait for each frame, so they have
    // no second batch to overlap: only a caller's context alternates.
    if (rc == 0) (*out)->ms_overlap = (*out)->own_stream;
    return rc;
}

void vqm_ctx_destroy(vqm_ctx *ctx) {
    DeviceScope scope;
    destroy(ctx);
}

int vqm_ssim_submit(vqm_ctx *ctx, const void *ref, const void *dis, int w, int h, int bpc) {
    DeviceScope scope;
    return submit(ctx, KIND_SSIM, &ref, &dis, 1, w, h, bpc, true);
}

int vqm_msssim_submit(vqm_ctx *ctx, const void *ref, const void *dis, int w, int h, int bpc) {
    DeviceScope scope;
    return submit(ctx, KIND_MSSSIM, &ref, &dis, 1, w, h, bpc, true);
}

int vqm_ssim_submit_batch(vqm_ctx *ctx, const void *const *refs, const void *const *dis, int n, int w, int h,
                          int bpc) {
    DeviceScope scope;
    return submit(ctx, KIND_SSIM, refs, dis, n, w, h, bpc, true);
}

int vqm_msssim_submit_batch(vqm_ctx *ctx, const void *const *refs, const void *const *dis, int n, int w, int h,
                            int bpc) {
    DeviceScope scope;
    return submit(ctx, KIND_MSSSIM, refs, dis, n, w, h, bpc, true);
}

int vqm_collect(vqm_ctx *ctx, double *score, double *lcs) {
    DeviceScope scope;
    return collect(ctx, score, lcs, nullptr);
}

int vqm_collect_db(vqm_ctx *ctx, double *score, double *db) {
    DeviceScope scope;
    return collect(ctx, score, nullptr, db);
}

int vqm_score_frames(vqm_ctx *const *ctxs, int nctx, int metric, const void *const *refs, const void *const *dis,
                     int n, int w, int h, int bpc, int batch, int lag, double *scores, double *lcs,
                     double *db) {
    DeviceScope scope;
    return score_frames(ctxs, nctx, metric, refs, dis, n, w, h, bpc, batch, lag, scores, lcs, db);
}

int vqm_in_flight(const vqm_ctx *ctx) { return ctx ? ctx->count : 0; }

int vqm_ctx_set_timing(vqm_ctx *ctx, int enable) {
    DeviceScope scope;
    if (!ctx) return fail(-EINVAL, "NULL context");
    int rc = ensure_device(ctx);
    if (rc) return rc;
    rc = drain_timing(ctx);
    if (rc) return rc;
    for (int i = 0; i < 4; ++i) {
        ctx->time_ms[i] = 0.0;
        ctx->launches[i] = 0;
        ctx->frames[i] = 0;
    }
    ctx->timing = enable != 0;
    return 0;
}

int vqm_ctx_kernel_time(vqm_ctx *ctx, int kernel_class, double *total_ms, int *launches, int *frames) {
    DeviceScope scope;
    if (!ctx) return fail(-EINVAL, "NULL context");
    if (kernel_class < 0 || kernel_class > 3) return fail(-EINVAL, "kernel class %d", kernel_class);
    int rc = ensure_device(ctx);
    if (rc) return rc;
    rc = drain_timing(ctx);
    if (rc) return rc;
    if (total_ms) *total_ms = ctx->time_ms[kernel_class];
    if (launches) *launches = ctx->launches[kernel_class];
    if (frames) *frames = ctx->frames[kernel_class];
    return 0;
}

int vqm_debug_decimate(vqm_ctx *ctx, const void *ref, const void *dis, int w, int h, int bpc, int scale,
                       float *out_ref, float *out_dis) {
    DeviceScope scope;
    if (!ctx || !out_ref || !out_dis) return fail(-EINVAL, "NULL argument");
    int rc = check_args(ref, dis, w, h, bpc);
    if (rc) return rc;
    if (scale == 0) {
        rc = gate_ssim(w, h, bpc, nullptr, nullptr, nullptr);
        if (rc) return rc;
    } else if (scale < 1 || scale > 128) {
        return fail(-EINVAL, "scale %d outside 1..128", scale);
    }
    Geometry g = make_geometry(KIND_SSIM, w, h, bpc);
    if (scale != 0 && scale != g.s) {
        // A forced scale is part of the slot's geometry key, so the next
        // automatic-scale frame rebuilds the slot.
        g.s = scale;
        g.dw = (w + scale - 1) / scale;
        g.dh = (h + scale - 1) / scale;
        g.dpitch = round_up(g.dw, 64);
    }
    rc = drain(ctx);
    if (rc) return rc;
    Slot *sl = nullptr;
    const void *dref = nullptr, *ddis = nullptr;
    rc = debug_slot(ctx, g, ref, dis, &sl, &dref, &ddis);
    if (rc) return rc;
    // A step launch with the decimation role only (scale 1 included: the
    // general path with tap 1 writes the sample values).
    vqm::StepRoles r;
    memset(&r, 0, sizeof r);
    r.n_dec = 1;
    r.dec.f[0].ref = dref;
    r.dec.f[0].dis = ddis;
    r.dec.f[0].out_ref = sl->planes + sl->off_ref[0];
    r.dec.f[0].out_dis = sl->planes + sl->off_dis[0];
    const vqm::StepGeometry sg = step_geometry(g);
    LAUNCH_TIMED(ctx, VQM_KERNEL_SSIM_STEP, 1,
                 vqm::launch_ssim_step(r, sg, sg.packed ? vqm::IN_U16 : vqm::IN_F32, g.dpitch,
                                       sg.packed ? sg.post : 1.0f, ctx->taps, ctx->stream, timer_));
    if (!sg.packed) {
        HIP_TRY(hipMemcpy2DAsync(out_ref, g.dw * sizeof(float), sl->planes + sl->off_ref[0],
                                 g.dpitch * sizeof(float), g.dw * sizeof(float), g.dh, hipMemcpyDeviceToHost,
                                 ctx->stream));
        HIP_TRY(hipMemcpy2DAsync(out_dis, g.dw * sizeof(float), sl->planes + sl->off_dis[0],
                                 g.dpitch * sizeof(float), g.dw * sizeof(float), g.dh, hipMemcpyDeviceToHost,
                                 ctx->stream));
        HIP_TRY(hipStreamSynchronize(ctx->stream));
        return 0;
    }
    // Packed planes hold the window sums: the value is sum * post, exact.
    std::vector<uint16_t> sums((size_t)g.dw * (size_t)g.dh * 2);
    uint16_t *hs[2] = {sums.data(), sums.data() + (size_t)g.dw * g.dh};
    const float *dev[2] = {sl->planes + sl->off_ref[0], sl->planes + sl->off_dis[0]};
    for (int i = 0; i < 2; ++i)
        HIP_TRY(hipMemcpy2DAsync(hs[i], g.dw * sizeof(uint16_t), dev[i], g.dpitch * sizeof(uint16_t),
                                 g.dw * sizeof(uint16_t), g.dh, hipMemcpyDeviceToHost, ctx->stream));
    HIP_TRY(hipStreamSynchronize(ctx->stream));
    float *outs[2] = {out_ref, out_dis};
    for (int i = 0; i < 2; ++i)
        for (size_t k = 0; k < (size_t)g.dw * g.dh; ++k) outs[i][k] = (float)hs[i][k] * sg.post;
    return 0;
}

int vqm_debug_pyramid(vqm_ctx *ctx, const void *ref, const void *dis, int w, int h, int bpc, int level,
                      float *out_ref, float *out_dis) {
    DeviceScope scope;
    if (!ctx || !out_ref || !out_dis) return fail(-EINVAL, "NULL argument");
    if (level < 2 || level > kLevels) return fail(-EINVAL, "pyramid level %d outside 2..5", level);
    int rc = check_args(ref, dis, w, h, bpc);
    if (rc) return rc;
    rc = gate_msssim(w, h);
    if (rc) return rc;
    const Geometry g = make_geometry(KIND_MSSSIM, w, h, bpc);
    rc = drain(ctx);
    if (rc) return rc;
    Slot *sl = nullptr;
    const void *dref = nullptr, *ddis = nullptr;
    rc = debug_slot(ctx, g, ref, dis, &sl, &dref, &ddis);
    if (rc) return rc;
    rc = enqueue_msssim(ctx, &sl, 1, &dref, &ddis, ctx->stream);
    if (rc) return rc;
    const int j = level - 1;
    HIP_TRY(hipMemcpy2DAsync(out_ref, g.lw[j] * sizeof(float), sl->planes + sl->off_ref[j],
                             g.lpitch[j] * sizeof(float), g.lw[j] * sizeof(float), g.lh[j], hipMemcpyDeviceToHost,
                             ctx->stream));
    HIP_TRY(hipMemcpy2DAsync(out_dis, g.lw[j] * sizeof(float), sl->planes + sl->off_dis[j],
                             g.lpitch[j] * sizeof(float), g.lw[j] * sizeof(float), g.lh[j], hipMemcpyDeviceToHost,
                             ctx->stream));
    HIP_TRY(hipStreamSynchronize(ctx->stream));
    return 0;
}

int vqm_debug_pyramid_batch(vqm_ctx *ctx, const void *const *refs, const void *const *dis, int n, int w, int h,
                            int bpc, int level, float *out_ref, float *out_dis) {
    DeviceScope scope;
    if (!ctx || !refs || !dis || !out_ref || !out_dis) return fail(-EINVAL, "NULL argument");
    if (n < 1 || n > VQM_MAX_BATCH) return fail(-EINVAL, "batch of %d frames outside 1..%d", n, VQM_MAX_BATCH);
    if (level < 2 || level > kLevels) return fail(-EINVAL, "pyramid level %d outside 2..5", level);
    int rc = 0;
    for (int i = 0; i < n; ++i) {
        rc = check_args(refs[i], dis[i], w, h, bpc);
        if (rc) return rc;
    }
    rc = gate_msssim(w, h);
    if (rc) return rc;
    const Geometry g = make_geometry(KIND_MSSSIM, w, h, bpc);
    rc = drain(ctx);
    if (rc) return rc;
    if (ctx->count + n > VQM_MAX_IN_FLIGHT)
        return fail(-EAGAIN, "%d frames in flight leave no room for %d more", ctx->count, n);
    rc = ensure_device(ctx);
    if (rc) return rc;
    Slot *sl[VQM_MAX_BATCH];
    const void *dref[VQM_MAX_BATCH], *ddis[VQM_MAX_BATCH];
    for (int i = 0; i < n; ++i) {
        Slot &s = ctx->slots[(ctx->head + ctx->count + i) % VQM_MAX_IN_FLIGHT];
        rc = prepare_slot(s, g);
        if (rc) return rc;
        rc = upload(ctx, s, refs[i], dis[i], &dref[i], &ddis[i]);
        if (rc) return rc;
        sl[i] = &s;
    }
    rc = enqueue_msssim(ctx, sl, n, dref, ddis, ctx->stream);
    if (rc) return rc;
    const int j = level - 1;
    const size_t plane = (size_t)g.lw[j] * (size_t)g.lh[j];
    for (int i = 0; i < n; ++i) {
        HIP_TRY(hipMemcpy2DAsync(out_ref + i * plane, g.lw[j] * sizeof(float), sl[i]->planes + sl[i]->off_ref[j],
                                 g.lpitch[j] * sizeof(float), g.lw[j] * sizeof(float), g.lh[j],
                                 hipMemcpyDeviceToHost, ctx->stream));
        HIP_TRY(hipMemcpy2DAsync(out_dis + i * plane, g.lw[j] * sizeof(float), sl[i]->planes + sl[i]->off_dis[j],
                                 g.lpitch[j] * sizeof(float), g.lw[j] * sizeof(float), g.lh[j],
                                 hipMemcpyDeviceToHost, ctx->stream));
    }
    HIP_TRY(hipStreamSynchronize(ctx->stream));
    return 0;
}

int vqm_ss2_channel_sums(const float *const *planes, int nch, int w, int h, double *sums) {
    return ss2_sums(planes, nch, w, h, sums);
}

int vqm_ss2_blur(const float *in, float *out, int w, int h, const float *coef) {
    return ss2_blur_plane(in, out, w, h, coef);
}

int vqm_ss2_downsample(const float *in, float *out, int w, int h) { return ss2_down_plane(in, out, w, h); }

int vqm_ss2_scale_sums(const float *const *ref, const float *const *dis, int nch, int w, int h, int nscales,
                       const float *coef, double *sums) {
    return ss2_chain(ref, dis, nch, w, h, nscales, coef, sums);
}

int vqm_ss2_cascade_coefficients(double sigma, float *coef) { return ss2_cascade(sigma, coef); }

int vqm_ss2_submit(vqm_ctx *ctx, const float *const *ref, const float *const *dis, int nch, int w, int h,
                   int nscales, const float *coef) {
    DeviceScope scope;
    return ss2_submit(ctx, ref, dis, nch, w, h, nscales, coef);
}

int vqm_ss2_collect(vqm_ctx *ctx, double *sums) {
    DeviceScope scope;
    return ss2_collect(ctx, sums);
}

int vqm_ss2_in_flight(const vqm_ctx *ctx) { return ctx ? ctx->ss2_count : 0; }

int vqm_debug_ss2_blurred(const float *const *ref, const float *const *dis, int nch, int w, int h, int nscales,
                          const float *coef, float *const *blurred, double *sums) {
    if (!blurred) return fail(-EINVAL, "NULL blurred-plane array");
    for (int c = 0; c < nch && c < vqm::kSs2MaxChannels; ++c)
        if (!blurred[c]) return fail(-EINVAL, "NULL blurred planes of channel %d", c);
    return ss2_chain(ref, dis, nch, w, h, nscales, coef, sums, blurred);
}

int vqm_debug_read_probe(const void *buf, long long bytes, int reps, double *ms) {
    return read_probe(buf, bytes, reps, ms);
}

int vqm_debug_valu_probe(int waves_per_simd, int iters, int reps, double *tflops) {
    return valu_probe(waves_per_simd, iters, reps, tflops);
}

int vqm_debug_pair_ops(int op, const float *a, const float *b, float *out, int n) {
    return pair_ops(op, a, b, out, n);
}

const char *vqm_last_error(void) { return g_err.c_str(); }

}  // extern "C"
