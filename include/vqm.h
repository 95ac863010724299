/*
 * vqm.h — C ABI of the MI355X (gfx950) per-frame float_ssim / MS-SSIM library.
 *
 * Sources (page title, section):
 *   [ADR-1405] "ADR-1405: float_ssim_hip decimates on the device,
 *              bit-identical to the CPU" — Context, Decision 1–4.
 *   [R-1363]   "Research-1363: Device-resident ssimulacra2 and a single-wait
 *              MS-SSIM on SYCL" — Findings 4 and 6.
 *   [ADR-1357] "ADR-1357: Run the SYCL CAMBI extractor entirely on the
 *              device" — Decision (one small result block read back per frame).
 *   [R-1369]   "Research-1369: SYCL psnr_hvs, motion_v2 and psnr at 4K" —
 *              §4 (pinned staging), §5 (slot fence), §7 (bit depths, sticky
 *              geometry).
 *
 * Conventions for every call:
 *   - Return 0 on success or a negative errno; never abort.  On error the
 *     output arguments are left untouched and vqm_last_error() holds a
 *     message for the calling thread.
 *       -EINVAL   NULL pointer; w or h <= 0; w*h above 2^31 - 1; bpc outside
 *                 8..16; an unusable stream or device index.
 *       -ENOTSUP  the frame is outside what the method defines: float_ssim
 *                 with scale > 128 or a decimated side < 11; MS-SSIM with
 *                 floor(w/16) < 11 or floor(h/16) < 11.  Checked on the host
 *                 before any HIP call ([ADR-1405] Decision 4).
 *       -ENOMEM   device or pinned-host allocation failed.
 *       -ENODEV   no HIP device.
 *       -EIO      a HIP runtime error (the message names it).
 *       -EAGAIN   vqm_collect with no frame in flight; a submit with
 *                 VQM_MAX_IN_FLIGHT frames already in flight.
 *       -ENOSPC   vqm_ssim_frame_noalloc: the frame needs more scratch than
 *                 its fixed array holds.
 *   - Planes are row-major and tightly packed (stride = w samples): uint8_t
 *     samples when bpc == 8, native-endian uint16_t with the value in the low
 *     bits when 9 <= bpc <= 16.  Samples above 2^bpc - 1 violate the
 *     contract: the call still returns and touches no memory outside its
 *     buffers, but the score is unspecified.
 *   - A plane pointer may be host pageable memory, host pinned memory
 *     (hipHostMalloc) or device memory on the context's device; the library
 *     tells them apart with hipPointerGetAttributes.  Pageable input is
 *     copied into pinned staging and sent with one DMA per plane; pinned
 *     input is sent directly; device input is read in place ([R-1369] §4).
 *   - The caller owns every buffer it passes.  The library owns its device
 *     scratch, pinned staging and result slots.
 *   - Ordering of device input: the library reads device planes on its own
 *     stream.  A stream the library creates for itself (the blocking calls',
 *     a context created with a NULL stream) is a blocking stream, so it
 *     starts after work already enqueued on the legacy default stream, which
 *     is where torch's default stream enqueues.  Planes written on any other
 *     stream must be complete before the call: synchronise with that stream
 *     first, or give that stream to vqm_ctx_create.
 *   - Read-back: a frame's result is one 8-byte double, written by the
 *     device straight into pinned host memory ([R-1363] Finding 6; the pages'
 *     one read-back per frame).  The decibel form (8 more bytes) and the 15
 *     MS-SSIM level means (120 more) cross only when a call asks for them.
 *
 * Numerics:
 *   - Every bit depth is mapped onto the 8-bit scale, v = raw * 2^-(bpc-8),
 *     so the SSIM constants use L = 255.
 *   - float_ssim: scale s = max(1, round(min(w,h)/256)); each plane is
 *     low-passed with an s x s box of fp32 weight 1.0f/(s*s) (formed on the
 *     host) and decimated to ceil(w/s) x ceil(h/s); every window sum is exact
 *     (an integer in units of 2^-52) and rounded once to fp32 — bit-identical
 *     to the plain definition; then the 11x11 Gaussian (sigma 1.5) SSIM map
 *     over the valid region, reduced to one double by a fixed-shape tree
 *     whose order depends only on the plane size ([ADR-1405] Context,
 *     Decision 1; [R-1363] Finding 4).
 *   - MS-SSIM: five levels at full resolution, level j+1 the exact 2x2 mean
 *     of level j; per level the means of luminance, contrast and structure
 *     (C3 = C2/2); MS = L5^b5 * prod_j (C_j S_j)^b_j with
 *     b = {0.0448, 0.2856, 0.3001, 0.2363, 0.1333}; NaN when any C_j or S_j
 *     is <= 0.  All five levels and the combine are enqueued at once and the
 *     host waits once per frame ([R-1363] Finding 6).  Each pixel's l, c, s
 *     terms are truncated to units of 2^-24 and summed exactly, so a level's
 *     means do not depend on the order of addition ([ADR-1357] Decision sums
 *     CAMBI's pool exactly in the same units).
 *   - Scores are bitwise repeatable for the same input on the same device,
 *     whatever the batch a frame is submitted in.
 */
#ifndef VQM_H
#define VQM_H

#ifdef __cplusplus
extern "C" {
#endif

#define VQM_ABI_VERSION 9

/* Exported symbols (the library is built with hidden default visibility). */
#if defined(__GNUC__)
#define VQM_API __attribute__((visibility("default")))
#else
#define VQM_API
#endif

/* Frames a context holds in flight between submit and collect: six full
 * batches, so a float_ssim batch's three pipeline stages can all be
 * enqueued before its frames are awaited. */
#define VQM_MAX_IN_FLIGHT 192

/* Frames one batched submit may hand over (processed per kernel launch).
 * Consecutive launches on one stream leave the GPU idle for a few
 * microseconds between them (the next kernel starts only once the last one
 * has drained); 32 frames per launch share that gap. */
#define VQM_MAX_BATCH 32

/* Number of per-level means vqm_msssim_frame_lcs returns: L_1..L_5,
 * C_1..C_5, S_1..S_5 ([R-1363] Finding 6, enable_lcs). */
#define VQM_MSSSIM_LCS 15

/* ssimulacra2 chain frames a context holds in flight between
 * vqm_ss2_submit and vqm_ss2_collect, each on a stream of its own. */
#define VQM_SS2_MAX_IN_FLIGHT 4

/* Device scratch, in bytes (8 MiB), of vqm_ssim_frame_noalloc: one array per GPU the
 * library runs on, held until the process ends. */
#define VQM_NOALLOC_SCRATCH_BYTES 8388608

/* ABI version of the loaded library (VQM_ABI_VERSION it was built with). */
VQM_API int vqm_abi_version(void);

/* Decimation factor max(1, round(min(w, h) / 256)) with real division and
 * ties away from zero ([ADR-1405] Context).  Pure host arithmetic; 0 when w
 * or h <= 0. */
VQM_API int vqm_ssim_scale(int w, int h);

/* Size of the decimated plane of a w x h frame (ceil(w/s) x ceil(h/s)) and
 * whether float_ssim accepts the frame: returns 0, or -EINVAL / -ENOTSUP as
 * vqm_ssim_frame would, without touching the GPU.  Any output may be NULL.
 * ([ADR-1405] Context: the scale rule; Decision 4: the gate refuses a
 * decimated plane below 11 x 11 or a scale above 128, nothing else.) */
VQM_API int vqm_ssim_geometry(int w, int h, int bpc, int *scale, int *dec_w, int *dec_h);

/* float_ssim of one frame pair, blocking ([ADR-1405] Context: decimate by
 * the automatic scale, then the SSIM map and its mean; Decision 1: exact
 * window sums; Decision 4: the gate; Context again: each frame is uploaded
 * once and read back once).  Runs on an idle library-owned context of the
 * current HIP device
 * (each with its own blocking stream; threads calling at once each get their
 * own, and the contexts are kept for later calls); one upload (unless the
 * planes are already on the device), one device wait, one 8-byte result.
 * *score receives the mean SSIM.  Thread-safe. */
VQM_API int vqm_ssim_frame(const void *ref, const void *dis, int w, int h, int bpc, double *score);

/* float_ssim plus its decibel form, blocking; as vqm_ssim_frame.  *db
 * receives -10 log10(1 - score), +inf when the score is 1 or more
 * ([ADR-1405] Consequences, enable_db: the form magnifies a score residual by
 * 4.34 / (1 - score) dB).  The finish kernel computes it beside the score;
 * the read-back is 16 bytes.  -EINVAL when db is NULL. */
VQM_API int vqm_ssim_frame_db(const void *ref, const void *dis, int w, int h, int bpc, double *score,
                              double *db);

/* 5-scale MS-SSIM of one frame pair, blocking; as vqm_ssim_frame.  All five
 * levels and the combine are enqueued together and the call waits once
 * ([R-1363] Finding 6: a partials span per scale, one wait per frame). */
VQM_API int vqm_msssim_frame(const void *ref, const void *dis, int w, int h, int bpc, double *score);

/* MS-SSIM plus the 15 per-level means (lcs: VQM_MSSSIM_LCS doubles, in the
 * order L_1..L_5, C_1..C_5, S_1..S_5). */
VQM_API int vqm_msssim_frame_lcs(const void *ref, const void *dis, int w, int h, int bpc,
                         double *score, double *lcs);

/* ---- Y'CbCr pictures: every plane scored ---- */

/* Chroma layouts.  Plane 0 is luma, w x h; planes 1 and 2 (Cb, Cr) are
 * halved horizontally in 4:2:0 and 4:2:2 and vertically in 4:2:0, an odd
 * size rounding up ((w + 1) / 2). */
enum vqm_chroma { VQM_CHROMA_420 = 0, VQM_CHROMA_422 = 1, VQM_CHROMA_444 = 2 };

/* Width and height of plane `plane` (0 = Y, 1 = Cb, 2 = Cr) of a w x h
 * picture in layout `chroma`.  Pure host; -EINVAL for bad arguments.
 * ([R-1363] Finding 6, enable_chroma; [R-1369] section 4.) */
VQM_API int vqm_plane_dims(int w, int h, int chroma, int plane, int *pw, int *ph);

/* float_ssim of each plane of a Y'CbCr frame pair ([R-1363] Finding 6,
 * enable_chroma): ref[p] and dis[p] are plane p (0 = Y, 1 = Cb, 2 = Cr),
 * tightly packed at the vqm_plane_dims size, each pointer of any kind
 * above.  Every plane is scored on its own (its own decimation scale);
 * scores[p] receives plane p's score and db (may be NULL) its decibel form.
 * The three planes are enqueued together and the call waits once.  Every
 * plane is checked and gated before anything is enqueued: -ENOTSUP when any
 * plane is refused (vqm_last_error names it). */
VQM_API int vqm_ssim_frame_yuv(const void *const *ref, const void *const *dis, int w, int h, int bpc, int chroma,
                               double *scores, double *db);

/* MS-SSIM of each plane, as vqm_ssim_frame_yuv; lcs (may be NULL) receives
 * 3 x VQM_MSSSIM_LCS doubles, plane by plane. */
VQM_API int vqm_msssim_frame_yuv(const void *const *ref, const void *const *dis, int w, int h, int bpc,
                                 int chroma, double *scores, double *lcs);

/* ---- explicit contexts: caller-chosen device and stream, pipelined ---- */

typedef struct vqm_ctx vqm_ctx;

/* Create a context on HIP device `device` ([R-1363] Finding 6: a twin's
 * submit() enqueues a frame and collect() waits once; [R-1369] §4–§5: the
 * pinned staging and the per-slot scratch such a context owns).  `hip_stream`
 * is a hipStream_t on that device to enqueue on (e.g.
 * torch.cuda.current_stream().cuda_stream), or NULL for a library-owned
 * blocking stream (see "Ordering of device input" above).  A context on a
 * library-owned stream runs every other MS-SSIM batch on a second stream of
 * its own, after the work already on the first (its uploads), so that one
 * batch's small levels run beside the next batch's first level; on a
 * caller's stream, in graph capture and with kernel timing on, every batch
 * stays on the one stream.  The stream must outlive the context.  A context
 * is not thread-safe: use one per thread.
 * Calls on a context make its device current while they run and restore the
 * calling thread's current device before they return. */
VQM_API int vqm_ctx_create(int device, void *hip_stream, vqm_ctx **out);

/* Wait for the context's frames, then free everything it owns.  NULL is a
 * no-op. */
VQM_API void vqm_ctx_destroy(vqm_ctx *ctx);

/* Enqueue one float_ssim frame (upload if needed, decimate, SSIM map,
 * fixed-tree reduction) and return without waiting ([R-1363] Finding 6:
 * submit() enqueues every stage; [R-1369] §4: pageable input through pinned
 * staging, one DMA; §5: a slot is reused only after its frame was collected;
 * §7: scratch keyed by the geometry).  Host pageable input is copied before
 * the call returns; pinned or device input must stay unchanged until the
 * matching vqm_collect.  Frames of different sizes may follow one another:
 * scratch is keyed by (w, h, bpc) and rebuilt when it changes.  The finish
 * also writes the decibel form, which vqm_collect_db may read. */
VQM_API int vqm_ssim_submit(vqm_ctx *ctx, const void *ref, const void *dis, int w, int h, int bpc);

/* Enqueue one MS-SSIM frame (all five levels and the combine; [R-1363]
 * Finding 6).  The finish also writes the 15 level means, which vqm_collect
 * may read. */
VQM_API int vqm_msssim_submit(vqm_ctx *ctx, const void *ref, const void *dis, int w, int h, int bpc);

/* Enqueue n (1..VQM_MAX_BATCH) frames of the same size and depth as one
 * batch: refs[i], dis[i] are frame i's planes (each pointer of any kind
 * above).  Every kernel of the path runs once for the whole batch, which
 * shares each launch's ramp-up, drain and the idle gap before the next
 * launch among n frames (at 2160p a lone frame's decimation spends a fifth
 * of its time there).  Each frame still
 * has its own upload, result slot and completion: collect them one by one,
 * in submission order, one wait each.  Needs n free in-flight slots
 * (-EAGAIN otherwise); nothing is enqueued on error. */
VQM_API int vqm_ssim_submit_batch(vqm_ctx *ctx, const void *const *refs, const void *const *dis, int n,
                                  int w, int h, int bpc);
VQM_API int vqm_msssim_submit_batch(vqm_ctx *ctx, const void *const *refs, const void *const *dis, int n,
                                    int w, int h, int bpc);

/* Wait for the oldest frame in flight (the one device wait of that frame,
 * [R-1363] Finding 6; [R-1369] §5: its slot is free again afterwards) and
 * return its score.  lcs (may be NULL) receives the 15 per-level means
 * when the frame was an MS-SSIM frame; for a float_ssim frame it is left
 * untouched. */
VQM_API int vqm_collect(vqm_ctx *ctx, double *score, double *lcs);

/* As vqm_collect, with the decibel form of a float_ssim frame's score in *db
 * (may be NULL; see vqm_ssim_frame_db).  An MS-SSIM frame has no decibel
 * form here: *db receives NaN. */
VQM_API int vqm_collect_db(vqm_ctx *ctx, double *score, double *db);

/* Number of frames in flight. */
VQM_API int vqm_in_flight(const vqm_ctx *ctx);

/* Metrics of vqm_score_frames. */
enum vqm_metric { VQM_METRIC_FLOAT_SSIM = 0, VQM_METRIC_MS_SSIM = 1 };

/* Score n frame pairs of one size and depth, pipelined, and block until all
 * are scored.  Frames go in batches of `batch` (1..VQM_MAX_BATCH) to the
 * nctx contexts in turn (for example one per device; on one device a
 * single context is fastest, since concurrent step kernels contend for the
 * same memory bandwidth); a frame is
 * collected — its one wait — once `lag` later frames have been submitted
 * (lag <= 0: 3 * batch, which keeps a float_ssim batch's three pipeline
 * stages enqueued before its result is awaited).  scores[i] receives frame i's score;
 * lcs (may be NULL) receives 15 doubles per frame for MS-SSIM;
 * db (may be NULL) receives each float_ssim frame's decibel form (NaN for
 * MS-SSIM).  The contexts
 * must have no frames in flight.  On error every submitted frame is still
 * collected before the call returns. */
VQM_API int vqm_score_frames(vqm_ctx *const *ctxs, int nctx, int metric, const void *const *refs,
                             const void *const *dis, int n, int w, int h, int bpc, int batch, int lag,
                             double *scores, double *lcs, double *db);

/* ---- recorded passes: one HIP graph replayed over a fixed set of frames ---- */

typedef struct vqm_graph vqm_graph;

/* Record one scoring pass over n (1..VQM_MAX_IN_FLIGHT) frame pairs as a HIP
 * graph on `device` and `hip_stream` (NULL: a stream of the graph's own):
 * for float_ssim the step launches of every batch of `batch`
 * (1..VQM_MAX_BATCH) frames and the pipeline's drain, for MS-SSIM the five
 * level launches and the combine of every batch
 * ([ADR-1357] Decision and Consequences: a frame's kernels registered once
 * with a combined graph, whose replay absorbs their launches; [R-1363]
 * Finding 6: one wait per pass).  refs[i], dis[i] must be device memory of
 * that device, w x h samples of bpc bits as in vqm_ssim_submit; the graph
 * keeps their addresses and reads whatever they hold when it is replayed.
 * The graph owns its scratch (n frame slots).  The same gate and argument
 * checks as a submit apply; on error nothing is recorded and *out is NULL. */
VQM_API int vqm_graph_create(int device, void *hip_stream, int metric, const void *const *refs,
                             const void *const *dis, int n, int w, int h, int bpc, int batch, vqm_graph **out);

/* Enqueue one replay of the recorded pass on the graph's stream and return
 * without waiting.  -EBUSY while the previous replay is not collected (a
 * replay overwrites the results of the last one). */
VQM_API int vqm_graph_launch(vqm_graph *g);

/* Wait for the replay (its one device wait) and read its n scores into
 * scores[0..n-1]; lcs (may be NULL) receives 15 doubles per frame for
 * MS-SSIM, db (may be NULL) each float_ssim frame's decibel form (NaN for
 * MS-SSIM).  -EAGAIN when no replay is in flight.  After it returns the
 * caller may overwrite the frames for the next replay. */
VQM_API int vqm_graph_collect(vqm_graph *g, double *scores, double *lcs, double *db);

/* Wait for the graph's stream, then free the graph and its scratch.  NULL is
 * a no-op. */
VQM_API void vqm_graph_destroy(vqm_graph *g);

/* ---- measurement and inspection ---- */

/* Turn per-kernel timing on or off: while on, every decimation, SSIM and
 * MS-SSIM level kernel is bracketed by HIP events on the context's stream.
 * Switching clears the accumulated times. */
VQM_API int vqm_ctx_set_timing(vqm_ctx *ctx, int enable);

/* Kernel classes reported by vqm_ctx_kernel_time.  A float_ssim "step"
 * launch decimates one batch while it maps the batch before and finishes the
 * one before that; its frame count is the frames it decimates.  "Drain"
 * launches only map and finish (the pipeline's tail, and every launch at
 * scale 1); their frame count is the frames they map. */
enum vqm_kernel_class {
    VQM_KERNEL_SSIM_STEP = 0,
    VQM_KERNEL_SSIM_DRAIN = 1,
    VQM_KERNEL_MSSSIM_LEVEL1 = 2,
    VQM_KERNEL_MSSSIM_COARSE = 3
};

/* Total milliseconds, launch count and frames processed by one kernel class
 * since timing was switched on (a batched launch counts once and processes
 * several frames).  Waits for the context's stream.  Any output may be NULL. */
VQM_API int vqm_ctx_kernel_time(vqm_ctx *ctx, int kernel_class, double *total_ms, int *launches,
                                int *frames);

/* Decimate one frame pair on the device with the float_ssim decimation
 * kernels and copy the two fp32 planes back (ceil(w/scale) x ceil(h/scale)
 * floats each, tightly packed).  scale = 0 picks the automatic scale and
 * applies the float_ssim gate, exactly as vqm_ssim_submit does; scale in
 * 1..128 forces that factor (the decimated plane may then be any size >= 1).
 * At scale 1 the planes are the sample values v.  Where the scoring path
 * keeps the decimated planes as 16-bit window sums (scale 2^k with
 * bpc + 2k <= 16), the kernels write those sums and this call returns them
 * times 2^-(2k + bpc - 8), which is exact.  Blocking.  For the
 * bit-exactness tests ([ADR-1405] Decision 2). */
VQM_API int vqm_debug_decimate(vqm_ctx *ctx, const void *ref, const void *dis, int w, int h, int bpc,
                               int scale, float *out_ref, float *out_dis);

/* Build the MS-SSIM pyramid on the device exactly as vqm_msssim_submit does
 * and copy level `level` (2..5, size floor(w/2^(level-1)) x
 * floor(h/2^(level-1))) of both planes back as fp32, tightly packed.  Level 1
 * is never materialised (its kernel reads the raw samples).  Blocking.  For
 * the bit-exactness tests of the pyramid. */
VQM_API int vqm_debug_pyramid(vqm_ctx *ctx, const void *ref, const void *dis, int w, int h, int bpc,
                      int level, float *out_ref, float *out_dis);

/* vqm_debug_pyramid for a batch of n frames (1..VQM_MAX_BATCH) of one size,
 * built in one launch per level exactly as vqm_msssim_submit_batch builds
 * them (so the level kernel a batch of that size takes runs): level `level` of
 * frame i is copied to out_ref + i * lw * lh and out_dis + i * lw * lh, with
 * lw x lh the level's size.  Blocking.  For the bit-exactness tests of the
 * pyramid. */
VQM_API int vqm_debug_pyramid_batch(vqm_ctx *ctx, const void *const *refs, const void *const *dis, int n, int w,
                                    int h, int bpc, int level, float *out_ref, float *out_dis);

/* ---- allocation-free float_ssim ---- */

/* float_ssim of one device-resident frame pair that allocates nothing, for
 * callers that cannot allocate: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It enqueues the same kernels as
 * vqm_ssim_frame (decimation, SSIM map, fixed-tree finish) on `hip_stream`
 * (a stream of the current device; NULL is the legacy default stream) and
 * returns without waiting: *score holds the frame's score once that stream's
 * work up to this call has completed.
 *   ref, dis   device memory of the current device, w x h samples of bpc bits
 *              as for vqm_ssim_frame; they must stay unchanged until the
 *              score is written.
 *   score      one double of device memory of the current device, or of
 *              pinned host memory (hipHostMalloc).
 * Scratch: a file-scope device array of VQM_NOALLOC_SCRATCH_BYTES per GPU
 * (both decimated planes and one double per 32 x 32 map tile), held until
 * the process ends.  Frames whose scratch exceeds it are refused with
 * -ENOSPC (every frame up to 8192 x 4320 fits; a decimated plane of about
 * a million samples does not).  Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (on different streams, or from
 * different threads without ordering) race and give unspecified scores.
 * Host memory planes are refused (-EINVAL), as are the gate's frames
 * (-ENOTSUP).  Makes no allocation of any kind; the first call on each device
 * takes the array's device address once. */
VQM_API int vqm_ssim_frame_noalloc(const void *ref, const void *dis, int w, int h, int bpc, double *score,
                                   void *hip_stream);

/* ---- ssimulacra2: the per-scale statistics on the device ---- */

/* The six ssimulacra2 sums of nch (1..3) channels at one scale, computed on
 * the device without fp64 and read back once ("Research-1363: Device-resident
 * ssimulacra2 and a single-wait MS-SSIM on SYCL", Findings 3-4).
 *   planes  7 * nch device pointers of the current device, channel by
 *           channel: img1, img2 (the two images), mu1, mu2 (their blurred
 *           means), s11, s22, s12 (the blurred products img1 img1, img2 img2,
 *           img1 img2); fp32, w x h, tightly packed.  Every pixel must have
 *           (s11 - mu1^2) + (s22 - mu2^2) + 0.0009 > 0 (true of any blur
 *           with non-negative weights, which keeps the variances >= 0).
 *   sums    6 * nch doubles (host memory): per channel
 *           { sum d, sum d^4, sum art, sum art^4, sum det, sum det^4 } with,
 *           per pixel, num_m = 1 - (mu1 - mu2)^2,
 *           num_s = 2 (s12 - mu1 mu2) + 0.0009, denom_s = (s11 - mu1^2) +
 *           (s22 - mu2^2) + 0.0009 (fp32, in this order),
 *           d = max(1 - num_m num_s / denom_s, 0),
 *           e = (1 + |img2 - mu2|) / (1 + |img1 - mu1|) - 1,
 *           art = max(e, 0), det = max(-e, 0).
 * Each term is an exact fp32 pair (two_prod, two-quotient ff_div, pair
 * products for the fourth powers) and each sum runs through a fixed tree —
 * a fixed strided subset of pixels per thread, a tree per workgroup, one
 * workgroup per channel over the partials — whose shape depends only on
 * w * h: the sums are bitwise repeatable and within about 1e-12 relative of
 * the exact sums.  Blocking: two launches on a library-owned blocking stream
 * and one wait.  -EINVAL for NULL pointers, a bad size or channel count, or
 * planes that are not device memory of the current device. */
VQM_API int vqm_ss2_channel_sums(const float *const *planes, int nch, int w, int h, double *sums);

/* The fp32-pair operations of vqm_ss2_channel_sums run elementwise on the
 * device, for the bit-exactness tests: out[i] = op(a[i], b[i]) over n
 * (1..2^24) pairs stored (hi, lo) interleaved in host arrays of 2n floats.
 * op: 0 two_sum(a.hi, b.hi), 1 two_prod(a.hi, b.hi), 2 ff_add, 3 ff_mul,
 * 4 ff_div.  Every step is a correctly rounded fp32 operation, so the
 * results are unique.  Blocking. */
VQM_API int vqm_debug_pair_ops(int op, const float *a, const float *b, float *out, int n);

/* ---- ssimulacra2: the per-scale chain on the device ---- */

/* The recursive blur of one w x h fp32 plane (tightly packed), the blur of
 * "Research-1363: Device-resident ssimulacra2 and a single-wait MS-SSIM on
 * SYCL", Findings 2 and 7: a sequential recursion along every row, then
 * along every column of the row pass's fp32 output.  The pages give no
 * coefficients; this is the third-order recursion with
 * coef = {B, a1, a2, a3} (host memory, finite), at rest outside the line,
 * causal then anticausal:
 *   w[i] = ((B x[i] + a3 w[i-3]) + a2 w[i-2]) + a1 w[i-1],   i = 0..n-1
 *   y[i] = ((B w[i] + a3 y[i+3]) + a2 y[i+2]) + a1 y[i+1],   i = n-1..0
 * each product rounded to fp32 on its own and the sum from the oldest state
 * to the newest, so the result is unique and bit-exact.
 *   in, out  device memory of the current device, w * h floats each; out
 *            may equal in (the blur then runs in place).
 * Blocking: two launches on a library-owned blocking stream and one wait.
 * -EINVAL for NULL pointers, a bad size, non-finite coefficients or planes
 * that are not device memory of the current device. */
VQM_API int vqm_ss2_blur(const float *in, float *out, int w, int h, const float *coef);

/* The 2x2 downsample between the chain's scales (Finding 7's "downsample"
 * stage; its form is a reading): a w x h plane to ceil(w/2) x ceil(h/2),
 * out = ((a + b) + (c + d)) * 0.25f over each 2x2 block (a, b its upper
 * row), the last column and row repeated when w or h is odd.  in, out:
 * device memory of the current device, tightly packed, not overlapping.
 * Blocking.  -EINVAL as vqm_ss2_blur. */
VQM_API int vqm_ss2_downsample(const float *in, float *out, int w, int h);

/* The ssimulacra2 per-scale chain of one frame, every scale on the device
 * and one wait (Finding 1's request of no round trips; Finding 7's stages
 * after the colour transform: three multiplies, horizontal and vertical
 * blur passes, the sums, the downsample).  For scale s = 0..nscales-1
 * (nscales 1..6) and channel c = 0..nch-1 (nch 1..3): a, b are ref[c],
 * dis[c] at s = 0 and the downsample of the previous scale's a, b after
 * that; the five planes a, b, a a, b b, a b go through vqm_ss2_blur's blur
 * with coef; and the six sums of vqm_ss2_channel_sums of
 * (a, b, blur(a), blur(b), blur(a a), blur(b b), blur(a b)) go to
 * sums[(s * nch + c) * 6 ..] (host memory, 6 * nch * nscales doubles).
 *   ref, dis  nch device pointers each (the current device), w x h fp32
 *             planes, tightly packed: the colour-transformed planes of the
 *             two pictures (the pages fix no constants of the transform, so
 *             it stays with the caller).
 *   coef      the recursion's four coefficients, as vqm_ss2_blur; a blur
 *             with a non-negative impulse response keeps every variance,
 *             and so the statistics' denominators, positive.
 * The multiplies, blurs and downsample are bit-exact; the sums are within
 * about 1e-12 relative of exact and bitwise repeatable.  The library keeps
 * a device workspace of about 5 * nch * w * h floats per blocking context
 * (and the smaller scales' images), grown on demand.  Blocking: four
 * launches for every scale together (the pyramid, the row pass, the column
 * pass with the statistics, the sums; three for one scale) on a
 * library-owned blocking stream and one wait.  -EINVAL for NULL pointers,
 * bad counts or sizes, non-finite coefficients or planes that are not
 * device memory of the current device; -ENOMEM when the workspace cannot
 * grow. */
VQM_API int vqm_ss2_scale_sums(const float *const *ref, const float *const *dis, int nch, int w, int h,
                               int nscales, const float *coef, double *sums);

/* vqm_ss2_scale_sums as a submit that does not wait ([R-1363] Finding 6:
 * submit() enqueues every stage, collect() waits once; Finding 1: the
 * frame's stages stay on the device).  The frame goes to the context's next
 * free chain slot (VQM_SS2_MAX_IN_FLIGHT of them), whose own stream waits
 * for the work already enqueued on the context's stream and then runs the
 * whole chain: frames in flight on one context overlap on the GPU, which a
 * lone frame's small later scales leave mostly idle.  Each slot keeps its
 * own workspace (as vqm_ss2_scale_sums's) and pinned result block, grown on
 * demand.  ref, dis must stay unchanged until the matching vqm_ss2_collect.
 * Arguments and errors as vqm_ss2_scale_sums (ref, dis on the context's
 * device), and -EAGAIN with VQM_SS2_MAX_IN_FLIGHT frames already in flight;
 * no frame is in flight after an error.  These slots are apart from the float_ssim
 * and MS-SSIM ones: vqm_collect never returns a chain frame. */
VQM_API int vqm_ss2_submit(vqm_ctx *ctx, const float *const *ref, const float *const *dis, int nch, int w, int h,
                           int nscales, const float *coef);

/* Wait for the oldest chain frame of the context (its one wait) and copy
 * its 6 * nch * nscales sums, laid out as vqm_ss2_scale_sums's, to `sums`
 * (host memory).  -EAGAIN when no chain frame is in flight. */
VQM_API int vqm_ss2_collect(vqm_ctx *ctx, double *sums);

/* Number of chain frames in flight on the context (0 for NULL). */
VQM_API int vqm_ss2_in_flight(const vqm_ctx *ctx);

/* Coefficients {B, a1, a2, a3} for the chain's blur whose impulse response
 * is a Gaussian-like bell of variance sigma^2 (0 < sigma < 1e6): three
 * symmetric exponential smoothers in series, B = (1 - p)^3, a1 = 3p,
 * a2 = -3p^2, a3 = p^3, with p in (0, 1) solving 6p / (1 - p)^2 = sigma^2.
 * One choice of recursive Gaussian among many (the pages name the filter,
 * not its coefficients); host arithmetic only.  -EINVAL for a NULL array or
 * sigma outside the range. */
VQM_API int vqm_ss2_cascade_coefficients(double sigma, float *coef);

/* vqm_ss2_scale_sums that also returns the five blurred planes its kernels
 * form at every scale, for the bit-exactness tests of "Research-1363:
 * Device-resident ssimulacra2 and a single-wait MS-SSIM on SYCL", Finding 2
 * (everything but the sums reproduces the CPU exactly).
 *   blurred  nch device pointers (the current device), each to
 *            5 * (w_0 h_0 + ... + w_{n-1} h_{n-1}) floats, w_s x h_s the
 *            size of scale s: per scale, in order, blur(a), blur(b),
 *            blur(a a), blur(b b), blur(a b) of the channel, tightly packed.
 *   sums     6 * nch * nscales doubles (host), as vqm_ss2_scale_sums.
 * Other arguments and errors as vqm_ss2_scale_sums; blocking. */
VQM_API int vqm_debug_ss2_blurred(const float *const *ref, const float *const *dis, int nch, int w, int h,
                                  int nscales, const float *coef, float *const *blurred, double *sums);

/* A streaming read of `bytes` (>= 16) of device memory `buf` with 16-byte
 * non-temporal loads, one workgroup of 256 threads per 64 KiB, timed
 * with HIP events around each of `reps` launches (after one untimed one);
 * *ms receives the mean kernel time.  The HBM read ceiling that the
 * decimation's loads can reach on this GPU, for the measurements beside the
 * published peak.  Blocking; allocates a small sink. */
VQM_API int vqm_debug_read_probe(const void *buf, long long bytes, int reps, double *ms);

/* The fp32 multiply-add rate of the GPU's vector units with ordinary
 * (non-packed) FMA instructions: waves_per_simd (1..32) waves of 64 lanes
 * per SIMD, each lane running 16 independent FMA chains for `iters`
 * (1..2^20) steps, timed with HIP events around each of `reps` launches
 * (after one untimed one); *tflops receives 2 x lane FMAs / mean kernel
 * time.  The ceiling of the arithmetic-bound kernels, for the measurements
 * beside the published fp32 vector peak.  Blocking; allocates one float per
 * thread. */
VQM_API int vqm_debug_valu_probe(int waves_per_simd, int iters, int reps, double *tflops);

/* Message of the last failed call on this thread ("" if none). */
VQM_API const char *vqm_last_error(void);

#ifdef __cplusplus
}
#endif
#endif
