/*
 * proj_add_rmsnorm.h -- C ABI of the MI355X (gfx950) projection -> residual add -> RMSNorm
 * library.
 *
 * The operation is the decoder-layer region that follows a row-parallel projection (o_proj or
 * down_proj): vLLM "TPSP Design" page, section 1 (Motivation: projection, then residual add
 * and normalisation) and section 3 (Fusion regions; Microchunk pipeline), for one device's
 * share with no collective.  For T tokens, projection input size K and hidden size H:
 *
 *     y[t,h]   = sum_k x[t,k] * W[h,k]                 (bf16 inputs, fp32 accumulation)
 *     r[t,h]  <- r[t,h] + y[t,h]                        (fp32 residual, updated in place)
 *     out[t,h] = r[t,h] / sqrt(mean_h r[t,:]^2 + eps) * g[h]   (fp32 math, one bf16 rounding)
 *
 * with g = w for standard RMSNorm (no bias, "TPSP Design" section 4 Constraints) and g = 1 + w
 * for the Gemma form (spyre-inference "Plugin Architecture" page, custom-op table, GemmaRMSNorm
 * row: the weight multiply is done in fp32).
 *
 * Conventions for every entry point below
 *  - Tensor pointers are DEVICE pointers on the current HIP device, row-major, 16-byte aligned.
 *  - bf16 tensors are passed as uint16_t bit patterns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls are
 *    asynchronous: they return once the work is enqueued on `stream`; the caller synchronises.
 *  - Shapes: K % 64 == 0 and H % 64 == 0 (an intermediate size that is not a multiple of 64 is
 *    zero-padded at load, which leaves the result unchanged: "Plugin Architecture" page,
 *    SiluAndMul row).  T >= 0; T == 0 is a successful no-op.
 *  - Return 0 (PR_OK) or a negative PR_ERR_* code; pr_last_error() gives a message.  Invalid
 *    arguments and HIP execution errors are returned to the caller; the library never retries
 *    or silently re-routes them ("TPSP Design" section 3, Profiling and fallback).  An
 *    execution failure found on the device after a call has returned (a single-launch wait
 *    that gave up, see proj_add_rmsnorm_single_launch) is returned as PR_ERR_HIP by the next
 *    call of any device entry point on that device, without any synchronisation.
 *  - HIP graph capture: the single launch can be captured (see there), and so can the
 *    conventional path once a call of the same or a larger shape has run on the device.  A
 *    call that would have to grow a library workspace while its stream is capturing returns
 *    PR_ERR_UNSUPPORTED before enqueuing anything, and so does every call that would run the
 *    microchunk pipeline (it records events and waits across a library stream).
 *  - Calls on one device are sequential: the library-owned workspace (pipeline slots, the
 *    borrowed output) is shared by all calls on that device, so concurrent calls from several
 *    host threads or streams on one device race ("TPSP Design" section 4: shared workspace
 *    assumes sequential invocation).
 */
#ifndef PROJ_ADD_RMSNORM_H
#define PROJ_ADD_RMSNORM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PR_VERSION 1

/* return codes */
#define PR_OK 0
#define PR_ERR_INVALID_ARG (-1) /* null pointer, negative size, bad enum, negative eps       */
#define PR_ERR_SHAPE (-2)       /* K or H not a multiple of 64, sizes too large                */
#define PR_ERR_MICROCHUNK (-3)  /* microchunk < 0 or > PR_MAX_MICROCHUNK                       */
#define PR_ERR_UNSUPPORTED (-4) /* call outside the tuned token range, no device, not gfx950   */
#define PR_ERR_NOMEM (-5)       /* workspace allocation failed                                 */
#define PR_ERR_HIP (-6)         /* a HIP call or kernel launch failed                          */

/* RMSNorm gain form */
#define PR_NORM_STANDARD 0 /* g = w      */
#define PR_NORM_GEMMA 1    /* g = 1 + w  */

/* source layouts accepted by pr_prepare_weight */
#define PR_WEIGHT_OUT_IN 0 /* nn.Linear layout W[H][K] ([out, in])                  */
#define PR_WEIGHT_IN_OUT 1 /* pre-transposed W^T[K][H] ([in, out], K rows of H)     */

/* microchunk cap in tokens ("TPSP Design" section 4 Constraints, Resources) */
#define PR_MAX_MICROCHUNK 4096

/* execution paths */
#define PR_PATH_CONVENTIONAL 0
#define PR_PATH_FUSED 1
#define PR_PATH_SINGLE 2 /* projection, add and norm in one launch */

/* Chunk value that stands for the single-launch fused path (pr_select, pr_set_tuning). */
#define PR_SINGLE_LAUNCH (-2)

/*
 * Weight preparation, once after the weights load ("TPSP Design" section 3, Profiling and
 * fallback: projection weights are prepared after load; "Plugin Architecture" page, section
 * Transposed linear weights: the layout change is paid once at load, not in every forward).
 *
 * W_src   [H][K] (PR_WEIGHT_OUT_IN) or [K][H] (PR_WEIGHT_IN_OUT) bf16, device, caller-owned.
 * W_prep  K*H bf16, device, caller-owned, written here.  Layout: the weight transposed to
 *         [in][out] order in groups of 8 input rows, W_prep[((k/8)*H + h)*8 + k%8] = W[h][k],
 *         so each output column's 8 consecutive k-values form one 16-byte matrix-core operand.
 *         This is the only weight layout proj_add_rmsnorm and proj_add_rmsnorm_unfused accept.
 * Must not alias W_src.  Errors: PR_ERR_INVALID_ARG, PR_ERR_SHAPE, PR_ERR_HIP.
 */
int pr_prepare_weight(const uint16_t* W_src, int src_layout, uint16_t* W_prep, int K, int H,
                      void* stream);

/*
 * SiluAndMul, the step before down_proj ("Plugin Architecture" page, SiluAndMul row and section
 * Fused projections stay fused: the merged gate/up projection returns [..., 2d] and SiluAndMul
 * slices gate and up out of it; the intermediate size is zero-padded to a multiple of 64 at
 * load, which is inert because silu(0) = 0).
 *
 * gate_up [T][2K] bf16, device, caller-owned: row t holds gate in columns [0, K) and up in
 *         [K, 2K) (the merged projection's output as it is laid out).
 * x       [T][K] bf16, device, caller-owned, written here: x = silu(gate) * up, computed in
 *         fp32 with silu(g) = g / (1 + e^-g) and rounded once to bf16 (round to nearest even).
 *         It is the x input of proj_add_rmsnorm and its siblings with the same K.
 * K is the padded intermediate size, a positive multiple of 64.  Both pointers 16-byte aligned;
 * x must not overlap gate_up.  Asynchronous on `stream`; T = 0 is a no-op.
 * Errors: PR_ERR_SHAPE, PR_ERR_INVALID_ARG, PR_ERR_UNSUPPORTED (not a gfx950 device), PR_ERR_HIP.
 */
int pr_silu_mul(const uint16_t* gate_up, uint16_t* x, int T, int K, void* stream);

/*
 * The fused region, one device's share ("TPSP Design" sections 1 and 3).
 *
 * x              [T][K] bf16, read only.
 * W              [K*H] bf16 prepared by pr_prepare_weight, read only.
 * residual_inout [T][H] fp32, read and updated in place: r += x . W^T.
 * norm_w         [H] fp32 (standard: gain w; Gemma: offset w, applied as 1 + w).
 * eps            >= 0, added to the mean square inside the square root.
 * microchunk     > 0: microchunked pipeline with chunks of this many tokens (<= 4096; a value
 *                  >= T gives one chunk).  Chunk i+1's projection overlaps chunk i's add+norm
 *                  on a second stream; three reusable fp32 slots guarded by readiness and
 *                  completion events hold the projection results; the rows past T in the last
 *                  chunk are padding and never update residual or output ("TPSP Design"
 *                  section 3, Microchunk pipeline).
 *                = 0: automatic: the tuned token threshold picks the pipeline (with the tuned
 *                  chunk size) when T >= threshold, else the conventional path.  Untuned shapes
 *                  and inconclusive tunings use the conventional path; a T above the largest
 *                  tuned token count returns PR_ERR_UNSUPPORTED ("TPSP Design" section 3,
 *                  Profiling and fallback; section 4, Resources).  The environment variables
 *                  PR_MICROCHUNK_TOKENS and PR_THRESHOLD_TOKENS override the tuned values; with
 *                  both set no tuning is needed.
 *                < 0: PR_ERR_MICROCHUNK.
 *                The pipeline cannot be captured in a HIP graph: on a capturing stream a call
 *                that selects it returns PR_ERR_UNSUPPORTED and enqueues nothing.
 * norm_kind      PR_NORM_STANDARD or PR_NORM_GEMMA.
 * out            [T][H] bf16, caller-owned, written.  NULL: the result goes to a library
 *                workspace returned by pr_workspace_output(), borrowed until the next call on
 *                this device ("TPSP Design" section 3: the output borrows a shared workspace
 *                and must be consumed before the next call).  Must not overlap x, W, the
 *                residual or norm_w; the residual must not overlap x, W or norm_w (byte ranges
 *                of the dense extents above; PR_ERR_INVALID_ARG otherwise).
 * stream         ordering stream (see conventions).
 */
int proj_add_rmsnorm(const uint16_t* x, const uint16_t* W, float* residual_inout,
                     const float* norm_w, float eps, int T, int K, int H, int microchunk,
                     int norm_kind, uint16_t* out, void* stream);

/*
 * Conventional path ("TPSP Design" section 1, "Conventional TP": projection, then the residual
 * add and norm), one device's share: one projection over all T tokens emitting y in bf16
 * (round to nearest even) to a library workspace, then one add+RMSNorm pass.  Same arguments
 * and ownership as proj_add_rmsnorm without `microchunk`.  Its result differs from the fused
 * path by the bf16 rounding of y.
 */
int proj_add_rmsnorm_unfused(const uint16_t* x, const uint16_t* W, float* residual_inout,
                             const float* norm_w, float eps, int T, int K, int H, int norm_kind,
                             uint16_t* out, void* stream);

/*
 * Single-launch fused path: the projection, residual add and RMSNorm of all T tokens in one
 * kernel launch.  It is the pipeline of proj_add_rmsnorm with its hand-offs moved into the
 * kernel ("TPSP Design" section 3, Microchunk pipeline: reusable slots guarded by readiness
 * and completion events): a chunk is one tile row of tokens, its slot is the tile's
 * accumulators, and its events are a per-tile-row completion counter and epoch-tagged partial
 * slots in device memory.  Each tile adds the residual to its fp32 projection result (the
 * fused semantics: y is not rounded), publishes per-token partial sums of squares, waits until
 * every tile of its row has published and then writes its part of the output.  The grid never
 * exceeds the workgroups the device holds at once and a wait only involves tiles of the same
 * round, so every wait ends once the launch's workgroups are placed.  A wait that nevertheless
 * exceeds its poll limit (about two seconds; another process holding CUs can cause it) gives
 * up: that tile writes neither its output rows nor its residual rows (the residual keeps its
 * value before the call, since every tile stores it only after its wait), a status bit read
 * by pr_device_status is set, and the next call of any device entry point on this device
 * returns PR_ERR_HIP (it reads a flag in host-mapped memory that the kernel sets; no
 * synchronisation is involved).
 *
 * Same arguments and ownership as proj_add_rmsnorm_unfused.  Requires H = tile columns * n
 * with n <= 64 for one of the tiles the library instantiates (256, 192 or 128 columns; the
 * 192 x 192 tile is this bf16 entry point's only, the FP8 and SiluAndMul forms take 256 or
 * 128 columns), else PR_ERR_SHAPE.  The result agrees with the fused pipeline within rounding (the sum of squares
 * is taken in another order).  Uses a device workspace of at most T * H / 128 64-bit slots
 * and 3 + T / 128 words (status, completion counters, and the launch epoch, which the kernel
 * itself advances), shared by all calls on the device (calls on one device are sequential,
 * as for every entry point).  A call allocates or clears workspace only when it needs more
 * than earlier calls did; once a call of the same or a larger shape has run on the device,
 * a call makes no allocation, fill or host synchronisation and can be captured in a HIP
 * graph on a non-null stream and replayed (each replay takes a fresh epoch on the device).
 *
 * A second form splits the K range of each 256 x 256 tile over a pair of workgroups, which
 * swap partial sums before the residual add (reached with the debug overrides
 * PR_FORCE_TILE=256x256 PR_FORCE_WAVES=8 PR_FORCE_SPLIT=2; never chosen by default, as it
 * measured slower).  It needs H a multiple of 256 and adds 64 MiB of exchange regions and
 * 4 * ceil(T / 256) * H / 256 64-bit words to the workspace; its results agree with the first
 * form within rounding.
 */
int proj_add_rmsnorm_single_launch(const uint16_t* x, const uint16_t* W, float* residual_inout,
                                   const float* norm_w, float eps, int T, int K, int H,
                                   int norm_kind, uint16_t* out, void* stream);

/*
 * The down_proj region from the merged gate/up projection output, in one launch: SiluAndMul
 * ("Plugin Architecture" page, SiluAndMul row: x = silu(gate) * up from the [..., 2d] output
 * of the merged projection) formed inside the projection's main loop, then the single launch's
 * residual add and RMSNorm.
 *
 * gate_up   [T][2K] bf16 as for pr_silu_mul (gate in columns [0, K), up in [K, 2K); K the
 *           padded intermediate size, zero-padded columns inert).
 * x is never written: each LDS stage of gate and up is converted in place to
 * x = bf16(silu(gate) * up) with the fp32 arithmetic of pr_silu_mul, so the result equals
 * pr_silu_mul followed by proj_add_rmsnorm_single_launch on the same tile configuration.
 * Every tile column of a row band converts the band's x again (H / tile columns times), which
 * the separate SiluAndMul pass does once.
 * W, residual_inout, norm_w, eps, norm_kind, out, stream: as proj_add_rmsnorm_single_launch,
 * with the same workspace, graph-capture and give-up behaviour and shape rules.
 * Errors: as proj_add_rmsnorm_single_launch.
 */
int proj_add_rmsnorm_silu(const uint16_t* gate_up, const uint16_t* W, float* residual_inout,
                          const float* norm_w, float eps, int T, int K, int H, int norm_kind,
                          uint16_t* out, void* stream);

/* ---------------------------------------------------------------------------------------- *
 * One rank's share under tensor parallelism, on one GPU ("TPSP Design" section 1 Motivation:
 * with a row-parallel projection each rank holds a slice of the input columns and of the
 * weight, its projection gives a partial sum of y, a reduce-scatter leaves each rank the
 * summed rows of its token shard, and each rank normalises about T/P tokens; section 3
 * Microchunk pipeline: the same per microchunk).  The collectives themselves are not part of
 * this library; these are the two computations on either side of them.
 * ---------------------------------------------------------------------------------------- */

/*
 * The rank's projection share: y_partial = x . W_slice^T with fp32 accumulation, unrounded.
 * x          [T][K] bf16: the rank's K input columns of the T tokens (K = the full input size /
 *            P), device, read.
 * W          the matching [H][K] column slice of the weight, prepared by pr_prepare_weight.
 * y_partial  [T][H] fp32, device, written (one plane: no K split inside the call).
 * K, H positive multiples of 64; 16-byte aligned; y_partial must not overlap x or W.
 * Asynchronous on `stream`; T = 0 is a no-op.  Errors: PR_ERR_SHAPE, PR_ERR_INVALID_ARG,
 * PR_ERR_HIP.
 */
int pr_project_partial(const uint16_t* x, const uint16_t* W, float* y_partial, int T, int K,
                       int H, void* stream);

/*
 * The owner's step after the reduce-scatter, for its `rows` tokens:
 *     r[t,h] <- r[t,h] + (partial_0 + partial_1 + ... + partial_{P-1})[t,h]  (fp32, rank order)
 *     out    =  RMSNorm(r) as for proj_add_rmsnorm.
 * partials        P planes of [rows][H] fp32, plane p at partials + p * plane_stride (elements;
 *                 plane_stride >= rows * H, a multiple of 4), device, read.
 * residual_inout  [rows][H] fp32 (the rank's token shard), read and updated in place.
 * norm_w, eps, norm_kind as proj_add_rmsnorm; out [rows][H] bf16 (not NULL).
 * The written buffers must not overlap the others.  Asynchronous on `stream`; rows = 0 is a
 * no-op.  Errors: PR_ERR_SHAPE, PR_ERR_INVALID_ARG, PR_ERR_HIP.
 */
int pr_add_rmsnorm_partials(const float* partials, int P, long long plane_stride,
                            float* residual_inout, const float* norm_w, float eps, int rows,
                            int H, int norm_kind, uint16_t* out, void* stream);

/* ---------------------------------------------------------------------------------------- *
 * FP8 projections ("TPSP Design" section 5 To-do: quantized projections, with their scales
 * handled across microchunks).  The format is OCP E4M3 (sign, 4 exponent bits with bias 7, 3
 * mantissa bits, no infinities, S.1111.111 the only NaN, largest finite 448), the format the
 * gfx950 matrix cores take for FP8.  Codes are passed as uint8_t.
 * ---------------------------------------------------------------------------------------- */

/*
 * Scaled E4M3 quantisation of a bf16 matrix by groups of rows.
 *
 * src     [rows][cols] bf16, device, read.
 * dst     [rows][cols] E4M3 codes, device, written.
 * scales  [ceil(rows / group_rows)] fp32, device, written: for the group of rows
 *         [g * group_rows, min(rows, (g + 1) * group_rows)), scale = largest |value| / 448 in
 *         fp32 (1 when the group is all zero).  Each code is value / scale (an fp32 division),
 *         rounded to the nearest E4M3 value with ties to even, magnitudes clamped to 448.
 *         Non-finite values follow the same definition: a group holding a NaN has a NaN scale
 *         and every code 0x7F; one holding an infinity (and no NaN) an infinite scale, codes
 *         +-0 for its finite values and 0x7F for the infinities.
 * Activations: group_rows = the microchunk (1 gives per-token scales).  A weight [H][K] with
 * one per-tensor scale: rows = H, cols = K, group_rows = H.
 * cols a positive multiple of 16; src, dst 16-byte aligned, scales 4-byte aligned; the three
 * must not overlap.  Groups of 1, 2 or 4 rows with cols <= 8192 are quantised in one pass over
 * the data; other calls take two passes and a library workspace of `rows` floats (grown; under
 * graph capture it must already be large enough).  Asynchronous on `stream`; rows = 0 is a
 * no-op.
 * Errors: PR_ERR_SHAPE, PR_ERR_INVALID_ARG, PR_ERR_UNSUPPORTED, PR_ERR_NOMEM, PR_ERR_HIP.
 */
int pr_quantize_fp8(const uint16_t* src, uint8_t* dst, float* scales, int rows, int cols,
                    int group_rows, void* stream);

/*
 * FP8 weight preparation, once after load: W_src E4M3 codes [H][K] (PR_WEIGHT_OUT_IN) or
 * [K][H] (PR_WEIGHT_IN_OUT) to W_prep[((k/16)*H + h)*16 + k%16] = W[h][k] (each output
 * column's 16 consecutive k-values form one 16-byte matrix-core operand).  K and H positive
 * multiples of 64; 16-byte aligned; no overlap.  Errors: PR_ERR_INVALID_ARG, PR_ERR_SHAPE,
 * PR_ERR_HIP.
 */
int pr_prepare_weight_fp8(const uint8_t* W_src, int src_layout, uint8_t* W_prep, int K, int H,
                          void* stream);

/*
 * The fused region with the FP8 projection, in the single-launch form (the pipeline's chunk
 * hand-offs inside one kernel, as proj_add_rmsnorm_single_launch):
 *
 *     y[t,h]  = x_scales[t / scale_rows] * w_scale[0] * sum_k dec(x_q[t,k]) * dec(W[h,k])
 *               (products exact, fp32 accumulation, the scale applied in fp32)
 *     r[t,h] <- r[t,h] + y[t,h];   out = RMSNorm(r) as for proj_add_rmsnorm.
 *
 * x_q       [T][K] E4M3 codes (pr_quantize_fp8 with group_rows = scale_rows).
 * x_scales  [ceil(T / scale_rows)] fp32 activation scales; scale_rows >= 1.
 * W_q       the weight prepared by pr_prepare_weight_fp8; w_scale: one fp32 on the device.
 * residual_inout, norm_w, eps, norm_kind, out, stream: as proj_add_rmsnorm_single_launch
 * (out NULL borrows the output workspace), with the same workspace, graph-capture and
 * give-up behaviour.  Same shape rules (K, H multiples of 64; H a multiple of the tile
 * columns).  Errors: as proj_add_rmsnorm_single_launch, plus PR_ERR_INVALID_ARG for
 * scale_rows < 1 or null or misaligned scale pointers.
 */
int proj_add_rmsnorm_fp8(const uint8_t* x_q, const float* x_scales, int scale_rows,
                         const uint8_t* W_q, const float* w_scale, float* residual_inout,
                         const float* norm_w, float eps, int T, int K, int H, int norm_kind,
                         uint16_t* out, void* stream);

/*
 * Library set-up on the current device: creates the device's library stream, events and the
 * host-mapped status flag, and looks up and clears the fixed workspace of
 * proj_add_rmsnorm_single_launch_noalloc (synchronises the device).  Every other entry point
 * sets itself up on first use; the no-allocation entry point requires this call once per
 * device beforehand.  Calling it again is a no-op.  Errors: PR_ERR_UNSUPPORTED (not a gfx950
 * device), PR_ERR_HIP.
 */
int pr_init(void);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): proj_add_rmsnorm_single_launch with its workspace
 * in a fixed device array of the library instead of a grown one.  The call allocates nothing
 * and fills nothing; it only enqueues the single-launch kernels on `stream`.
 *
 * Same arguments, semantics and result as proj_add_rmsnorm_single_launch (the same kernels and
 * configuration; the result is bitwise equal), except:
 *  - pr_init() must have been called on the current device (else PR_ERR_UNSUPPORTED);
 *  - out must not be NULL (a borrowed output would be allocated): PR_ERR_INVALID_ARG;
 *  - the fixed array holds 2^20 64-bit row slots (8 MiB) and 4096 32-bit words per device:
 *    a launch needs min(T, rows per launch) * H / (tile columns) slots and 3 + tile rows words,
 *    so with 128-column tiles T * H <= 2^27 (T = 32768 at H = 4096) and with 256-column tiles
 *    T * H <= 2^28 (T = 32768 at H = 8192); a larger call returns PR_ERR_SHAPE before
 *    enqueuing anything.  The K-split pair form (a debug override) is not available:
 *    PR_ERR_UNSUPPORTED.
 *  - every call on a device shares that device's array, which keeps the last call's contents
 *    (epoch-tagged slots; each launch returns its completion counters to zero), so calls that
 *    overlap on one device race: enqueue them on one stream or order them.
 * No timing events are recorded for it (pr_profile_enable does not see it).  A wait that gives
 * up is reported as for the single launch (pr_device_status covers the fixed array too).
 */
int proj_add_rmsnorm_single_launch_noalloc(const uint16_t* x, const uint16_t* W,
                                           float* residual_inout, const float* norm_w, float eps,
                                           int T, int K, int H, int norm_kind, uint16_t* out,
                                           void* stream);

/*
 * Status bits that single-launch calls on the current device collected since the last read:
 * bit 0 = a tile's wait for its row gave up (its output and residual rows are not written).
 * Waits for the calls enqueued on `stream` to finish, stores the bits in *status (0 when
 * none) and clears them, together with the host-side flag the next call would report.
 * Errors: PR_ERR_INVALID_ARG (status NULL), PR_ERR_HIP.
 */
int pr_device_status(void* stream, unsigned* status);

/* Device pointer of the borrowed output of the last call made with out == NULL on the current
 * device, or NULL if there was none.  Valid until the next call on that device. */
const uint16_t* pr_workspace_output(void);

/*
 * Frees every workspace the library has grown on the current device (pipeline slots, the
 * conventional path's projection output, the borrowed output, the single launch's slots and
 * words, the pair form's exchange regions) after waiting for all work on the device; the
 * library stream and events stay.  The next call grows what it needs again ("TPSP Design"
 * section 4, Resources: the workspace is sized by the largest microchunk and token count
 * used).  The borrowed output pointer becomes invalid.  Not to be called while another call on
 * the device is in flight.  Errors: PR_ERR_UNSUPPORTED (no usable device), PR_ERR_HIP.
 */
int pr_release_workspace(void);

/* ---------------------------------------------------------------------------------------- *
 * Host-only helpers (no device work; usable without a GPU)
 * ---------------------------------------------------------------------------------------- */

/* Argument checks of proj_add_rmsnorm (pointers are checked for NULL, alignment and overlap of
 * the written buffers with the others; nothing is dereferenced). */
int pr_validate(const void* x, const void* W, const void* residual_inout, const void* norm_w,
                float eps, int T, int K, int H, int microchunk, int norm_kind, const void* out);

/* Argument checks of proj_add_rmsnorm_silu (gate_up holds 4 * T * K bytes). */
int pr_validate_silu(const void* gate_up, const void* W, const void* residual_inout,
                     const void* norm_w, float eps, int T, int K, int H, int norm_kind,
                     const void* out);

/* Argument checks of proj_add_rmsnorm_fp8 (x_q and W_q hold one byte per element; the scale
 * pointers must be non-null and 4-byte aligned and must not overlap the written buffers). */
int pr_validate_fp8(const void* x_q, const void* x_scales, int scale_rows, const void* W_q,
                    const void* w_scale, const void* residual_inout, const void* norm_w,
                    float eps, int T, int K, int H, int norm_kind, const void* out);

/* Execution decision for one call. */
typedef struct {
  int path;       /* PR_PATH_FUSED, PR_PATH_CONVENTIONAL or PR_PATH_SINGLE          */
  int microchunk; /* chunk tokens (fused), else T                                   */
  int n_chunks;   /* ceil(T / microchunk) (fused), else 1                           */
  int last_valid; /* valid rows of the last chunk                                   */
  int gemm_bm;    /* projection tile rows                                           */
  int gemm_bn;    /* projection tile columns                                        */
  int split_k;    /* K partitions of the projection; partial sums are added in order */
  int gemm_waves; /* waves per projection workgroup (4 or 8)                         */
  int reason;     /* PR_REASON_*                                                    */
  int gemm_stages; /* LDS ring depth of the projection (0 = the tile's default)      */
  int gemm_kgroups; /* K groups inside a projection workgroup (1, or 2 for the single
                       launch's 256x128 tile with 8 waves: two groups of 4 waves each
                       computing the tile over alternate 32-deep halves of K)          */
  int addnorm_cus;  /* fused pipeline: CUs reserved for the add/norm stream (the
                       CU-partitioned schedule of pr_plan_cu_split); 0 = the two-stream
                       ping-pong schedule of pr_plan                                    */
} pr_decision;

#define PR_REASON_EXPLICIT 0          /* microchunk > 0 given by the caller            */
#define PR_REASON_ABOVE_THRESHOLD 1   /* auto: T >= tuned/override threshold          */
#define PR_REASON_BELOW_THRESHOLD 2   /* auto: T < threshold                          */
#define PR_REASON_UNTUNED 3           /* auto: no tuning for this shape               */
#define PR_REASON_INCONCLUSIVE 4      /* auto: tuning found no profitable range       */
#define PR_REASON_UNFUSED_CALL 5      /* proj_add_rmsnorm_unfused                      */
#define PR_REASON_SINGLE_CALL 6       /* proj_add_rmsnorm_single_launch                */

/* Decision proj_add_rmsnorm would take (microchunk as in proj_add_rmsnorm; -1 = the unfused
 * entry point, PR_SINGLE_LAUNCH = the single-launch entry point).  Returns PR_OK or the error
 * that call would return. */
int pr_select(int T, int K, int H, int microchunk, pr_decision* d);

/* Dry-run schedule of the microchunk pipeline: the ordered list of operations the library
 * enqueues for T tokens and chunk size mc (host order).  Chunks alternate between the caller's
 * stream (even chunks) and a library stream (odd chunks); a chunk's projection and its add/norm
 * are consecutive on one stream, so chunk c+1's projection on the other stream overlaps chunk
 * c's add/norm.  On the host, chunk c+1's projection is enqueued before chunk c's add/norm so
 * that it reaches its stream while chunk c's projection still runs.  Slot c % 3 is reused by
 * chunk c+3, which runs on the other stream and waits for done[slot]; done[slot] is recorded
 * only where something waits for it, and a record that
 * follows the launch it marks is signalled by that launch.  The library stream starts after
 * the caller's prior work (entry event) and the caller's stream waits for the library stream's
 * last chunk (join).  Returns the number of operations (written up to max_ops), or a negative
 * error. */
typedef struct {
  int op;     /* PR_OP_*                                  */
  int stream; /* 0 = caller's stream, 1 = library stream  */
  int chunk;  /* chunk index or -1                        */
  int slot;   /* slot / event index (chunk % 3) or -1     */
  int rows;   /* valid rows of the chunk or 0             */
} pr_plan_op;

#define PR_OP_RECORD_ENTRY 0 /* caller stream: record the entry event                      */
#define PR_OP_WAIT_ENTRY 1   /* library stream: wait for the entry event                    */
#define PR_OP_WAIT_DONE 2    /* wait done[slot] (chunk c-3, other stream) before reusing it */
#define PR_OP_GEMM 3         /* projection of the chunk into slot                           */
#define PR_OP_ADDNORM 4      /* residual add + RMSNorm of the chunk from slot               */
#define PR_OP_RECORD_DONE 5  /* record done[slot] after the chunk's add/norm               */
#define PR_OP_JOIN 6         /* caller stream: wait done[slot] of the library stream's last */
#define PR_OP_WAIT_PREV 7    /* caller stream: wait for the previous call's last chunks when
                                that call was made on a different caller stream            */
#define PR_OP_RECORD_READY 8 /* record ready[slot] after the chunk's projection             */
#define PR_OP_WAIT_READY 9   /* wait ready[slot] before the chunk's add/norm                */
#define PR_NUM_SLOTS 3

int pr_plan(int T, int microchunk, pr_plan_op* ops, int max_ops);

/*
 * Dry-run schedule of the CU-partitioned pipeline ("TPSP Design" section 3, Profiling and
 * fallback: the microchunk size is tuned together with SM-count targets; on MI355X the target
 * is a CU mask on each stream).  Stream 1 is a library stream restricted to the projection's
 * CUs and runs every chunk's projection; stream 2 is a library stream restricted to the CUs
 * reserved for the add/norm and runs every chunk's add/norm, so chunk c+1's projection and
 * chunk c's add/norm run on disjoint CUs at the same time.  Slot s = c % 3: the projection
 * records ready[s], the add/norm waits for it and records done[s], and chunk c+3's projection
 * waits for done[s] before it overwrites the slot.  Both streams start after the caller's
 * prior work (entry event) and the caller's stream waits for the last chunk's done (join).
 * Same return convention as pr_plan; stream ids 0 (caller), 1 and 2.
 */
int pr_plan_cu_split(int T, int microchunk, pr_plan_op* ops, int max_ops);

/* ---------------------------------------------------------------------------------------- *
 * Token-threshold tuning ("TPSP Design" section 3, Profiling and fallback)
 * ---------------------------------------------------------------------------------------- */

/*
 * Threshold from measured timings, summed over shape groups (host-only).
 * t_conv, t_fused: [ngroups][nT] median seconds (t_fused = best checked chunk size; <= 0 when
 * no candidate passed the numerical check).  spread: [ngroups][nT] run-to-run spread
 * (p90 - p10) of the fused timing, or NULL.  T_grid ascending.  The threshold is the smallest
 * grid T such that at it and at every larger grid T the summed fused time beats the summed
 * conventional time by more than max(2%, summed spread); *threshold = INT32_MAX when none
 * (inconclusive: the conventional path is kept).
 */
int pr_threshold_from_timings(int ngroups, int nT, const int* T_grid, const double* t_conv,
                              const double* t_fused, const double* spread, int* threshold);

/* Install a tuning result for the shape group (K, H): fused iff T >= threshold_tokens with
 * chunk size mc_for_T[i] for T in [T_grid[i], T_grid[i+1]) (PR_SINGLE_LAUNCH: the
 * single-launch path); calls with T > max_tokens fail with PR_ERR_UNSUPPORTED.
 * threshold_tokens = INT32_MAX marks an inconclusive tuning. */
int pr_set_tuning(int K, int H, int threshold_tokens, int max_tokens, const int* T_grid,
                  const int* mc_for_T, int nT);

/* Install the projection configuration used for the chunks of every fused call of the shape
 * group (K, H) with this microchunk (explicit or auto): tile tile_m x tile_n (256x256, 256x128
 * or 128x128), split_k K partitions (split_k divides K/64), waves 4 or 8 per workgroup.  This
 * is the MI355X form of the SM-count targets the "TPSP Design" page tunes per group next to
 * the chunk size (section 3, Profiling and fallback): the tile and K split fix how many CUs a
 * chunk's projection occupies while the neighbouring chunk's projection and add/norm share the
 * GPU.  pr_tune installs these; without one, a time model chooses.  The result changes only
 * by summation order (within the parity tolerance).  Errors: PR_ERR_SHAPE, PR_ERR_MICROCHUNK,
 * PR_ERR_INVALID_ARG. */
int pr_set_chunk_config(int K, int H, int microchunk, int tile_m, int tile_n, int split_k,
                        int waves);

/* Install the CU split of the fused pipeline for the shape group (K, H) with this microchunk:
 * addnorm_cus CUs (a multiple of 8 from 8 to 128, spread evenly over the 8 XCDs) run the
 * add/norms and the other CUs the projections, on two CU-masked library streams
 * (pr_plan_cu_split); 0 selects the two-stream ping-pong schedule of pr_plan.  The chunk's
 * projection configuration is kept (the time model's when none was installed).  The result is
 * bitwise the same for every split (same kernels, same configurations).  Errors:
 * PR_ERR_SHAPE, PR_ERR_MICROCHUNK, PR_ERR_INVALID_ARG. */
int pr_set_cu_split(int K, int H, int microchunk, int addnorm_cus);

/* Remove every installed tuning result and chunk configuration. */
void pr_clear_tuning(void);

/*
 * Tuning results across processes: the page tunes once per shape group and keeps the result
 * ("TPSP Design" section 3, Profiling and fallback); these keep it past the process.
 * pr_tuning_save writes every installed tuning result and chunk configuration to the text file
 * `path` (replacing it), under a header naming the library version and a device key.
 * pr_tuning_load reads such a file and installs its records (replacing installed ones of the
 * same shape group and chunk size, keeping the others); a file of another library version or
 * device key is refused (PR_ERR_UNSUPPORTED) and a malformed or invalid record fails the whole
 * load (PR_ERR_INVALID_ARG, or the setter's code), leaving the installed tables as they were.
 * device_key NULL means the current device ("<gcnArchName>:<CU count>", which needs a device);
 * a caller may pass its own key (no white space).  Host-only apart from that device query.
 */
int pr_tuning_save(const char* path, const char* device_key);
int pr_tuning_load(const char* path, const char* device_key);

typedef struct {
  int threshold_tokens; /* INT32_MAX when inconclusive                         */
  int max_tokens;
  int n_checked;        /* candidate configurations that passed the check      */
  int n_rejected;       /* candidates that failed the numerical check          */
} pr_tune_report;

/*
 * Autotune on the current device: for each group g (shape K[g] x H[g]) and each T in T_grid,
 * time the conventional path, the pipeline for every chunk size in mc_cand (<= min(T, 4096))
 * and the single-launch path (when H allows it); the fused candidates are the pipeline chunk
 * sizes and the single launch, and the best of them is the fused time at T.  Each candidate's
 * result is first checked against the conventional path's result and dropped if it fails:
 * output relative L2 <= 5e-3 and per element |delta| <= 2e-2 + one bf16 ulp (both outputs are
 * rounded); residual per element within half a bf16 ulp of y plus fp32 rounding (the paths
 * differ exactly by the bf16 rounding of y).  At each T the conventional path and the candidates
 * that pass are timed round-robin (one call each per round, max(reps, 5) rounds after a
 * warm-up round; the chip's clock drifts with its power state, so back-to-back series would
 * favour whichever ran first) and each is represented by its median, on synthetic device data.  Before that, for each group and chunk size, the projection configurations of
 * the chunks are chosen: the time model's three best tile/split choices for a chunk alone on
 * the GPU and its three best with half the GPU (the other stream's chunk runs alongside), each
 * with 8 and 4 waves, are checked and timed round-robin in the pipeline at
 * T = min(max T_grid, 4 x chunk size), and the fastest that passes is installed with
 * pr_set_chunk_config, the model's first choice standing unless beaten by more than 3%; then,
 * with that configuration, the CU split of the chunk size (the page tunes SM-count targets
 * jointly with the microchunk): the ping-pong schedule and the CU-partitioned one with 32 and
 * 64 CUs reserved for the add/norms are checked and timed round-robin at the same T, and a
 * split is installed with pr_set_cu_split only if it beats the ping-pong schedule by more than
 * 3% (both steps skipped when a PR_FORCE_* override is set).  Installs the result with pr_set_tuning for
 * every group (chunk value PR_SINGLE_LAUNCH where the single launch is the fastest fused
 * candidate).  timings_out (optional): [ngroups][nT][3 + nmc] seconds: conventional, best
 * fused, each chunk size in mc_cand order, then the single launch; <= 0 for skipped or
 * rejected candidates.  With PR_MICROCHUNK_TOKENS and PR_THRESHOLD_TOKENS both set, nothing is
 * timed or checked and the override is installed.
 */
int pr_tune(const int* K, const int* H, int ngroups, int norm_kind, const int* T_grid, int nT,
            const int* mc_cand, int nmc, int reps, pr_tune_report* report, double* timings_out,
            void* stream);

/* ---------------------------------------------------------------------------------------- *
 * Kernel timing for benchmarks: while enabled, every projection and add/norm launch of the
 * calls on the current device is bracketed by timing events on the stream it runs on (the
 * library's pipeline streams or the caller's stream).  pr_profile_read waits for the recorded
 * events and returns the summed durations; the counters restart at every pr_profile_enable.
 * ---------------------------------------------------------------------------------------- */
typedef struct {
  double gemm_ms;       /* summed duration of projection launches           */
  int gemm_launches;
  double addnorm_ms;    /* summed duration of add + RMSNorm launches        */
  int addnorm_launches;
} pr_profile;

int pr_profile_enable(int on);
int pr_profile_read(pr_profile* p);

/* ---------------------------------------------------------------------------------------- */
const char* pr_strerror(int code);
const char* pr_last_error(void); /* message of the last failing call on this host thread */
int pr_version(void);

#ifdef __cplusplus
}
#endif
#endif /* PROJ_ADD_RMSNORM_H */
