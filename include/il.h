/*
 * il.h -- C ABI of the MI355X (gfx950) accelerator linear layer.
 *
 * One operation: a batch of matmuls that share one f32 input,
 *
 *     for every job j:   y_j[t][n_out_j] = x[t][n_in] * W_j^T
 *
 * (oxinfer 0.0.0 `src/gpu.rs` page: the doc comment of `struct Job` states
 * the product; `trait Backend` gives the calls `wants`, `upload`, `matmul`,
 * `name` and `stats` that the functions below follow).  Each W_j is
 * `[n_out, n_in]` row-major, stored as bf16, Q8 or Q4 (`enum WeightRef` on
 * the same page).  The pages do not show the Q8/Q4 layouts (`QMatrix`,
 * `Q4Matrix` are imported but not printed), so this library fixes them as
 * described at IL_Q8 / IL_Q4.
 *
 * Conventions for every function:
 *   - sizes are int64_t; all multi-byte fields are little-endian;
 *   - functions never print; on failure they set a thread-local message
 *     readable with il_last_error();
 *   - every function is thread-safe (`trait Backend: Send + Sync`).  The
 *     device context is created once per process on first use, on the HIP
 *     device current at that moment.
 */
#ifndef IL_H
#define IL_H

#include <stdint.h>

#if defined(__GNUC__)
#define IL_API __attribute__((visibility("default")))
#else
#define IL_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Storage format of a weight (`enum WeightRef`). */
typedef enum {
    /* uint16_t[n_out][n_in]: raw bfloat16 bits (WeightRef::Bf16(&[u16])). */
    IL_BF16 = 0,
    /* n_out * (n_in/32) packed 36-byte blocks, row-major by (row, block):
     *   { float32 scale; int8 q[32]; }   value of element e = q[e] * scale
     * (symmetric int8 with one f32 scale per 32-element block). */
    IL_Q8 = 1,
    /* n_out * (n_in/32) packed 18-byte blocks, row-major by (row, block):
     *   { uint16 scale_f16_bits; uint8 qs[16]; }
     * element 2j is the low nibble of qs[j], element 2j+1 the high nibble;
     * value of element e = (code[e] - 8) * f16(scale)  (4-bit, offset 8). */
    IL_Q4 = 2
} il_fmt;

/* Opaque device state of one uploaded weight (`type DeviceWeight`, "owned
 * by the layer"): immutable after il_upload, so concurrent il_matmul calls
 * may share it.  Freed with il_free. */
typedef struct il_weight il_weight;

/* One matmul of a batch (`struct Job`): y[t][n_out] = x[t][n_in] * W^T.
 *   w     : handle from il_upload; its n_in must equal il_matmul's n_in.
 *   n_out : must equal the handle's n_out.
 *   y     : DEVICE pointer to float[t][n_out] row-major, written in full
 *           (every element, once).  The y buffers of one call must not
 *           overlap each other or x. */
typedef struct {
    const il_weight *w;
    int64_t n_out;
    float *y;
} il_job;

/* Backend::upload -- prepare device state for one weight.
 *   weight : HOST pointer to the weight in format `fmt` (see il_fmt); it is
 *            borrowed for the duration of the call and copied, so the caller
 *            may free it on return.
 *   n_out, n_in : the weight's shape; n_out >= 1, n_in >= 32 and
 *            n_in % 32 == 0 (the Q8/Q4 block size; required for every
 *            format).
 * Copies the bytes to HBM and rearranges them into the device layout
 * (code plane + scale plane for Q8/Q4).  Synchronous: the handle is ready on
 * return.  Returns NULL on failure ("declined", the page's `None`): bad
 * fmt or shape, null pointer, no HIP device, out of device memory; the
 * reason is in il_last_error(). */
IL_API il_weight *il_upload(const void *weight, il_fmt fmt, int64_t n_out, int64_t n_in);

/* Element type of the full-precision weights given to il_upload_quantize. */
typedef enum {
    IL_SRC_F32 = 0,  /* float[n_out][n_in] */
    IL_SRC_BF16 = 1  /* uint16_t[n_out][n_in], raw bfloat16 bits */
} il_src;

/* Quantise on upload -- builds a Q8 or Q4 weight on the device from
 * full-precision weights (the step before `enum WeightRef`'s Q8 / Q4 on the
 * oxinfer 0.0.0 src/gpu.rs page: constructing the QMatrix / Q4Matrix that
 * page imports; the README page's "quantized weights").  The pages do not
 * show the quantiser, so this library's rule is symmetric absmax scaling per
 * 32-element block of a row, with amax = max |w| over the block:
 *   IL_Q8: s = amax / 127 (f32 division); q = rint(w / s) clamped to
 *          [-127, 127]; the block stores s as f32;
 *   IL_Q4: s = amax / 7 (f32 division) rounded to the nearest binary16 (ties
 *          to even), saturated at 65504; code = rint(w / s) clamped to
 *          [-8, 7], plus 8, where s is the stored binary16 value;
 *   a zero scale stores 0 and all-zero values (Q8 code 0, Q4 code 8).
 * rint rounds half to even; every division is correctly rounded.
 *   weight : HOST or DEVICE pointer (on the current device) to n_out * n_in
 *            elements of type `src`, row-major; borrowed for the call (a
 *            host buffer is copied to the device first).  Device contents
 *            must be complete when the call starts (synchronize the stream
 *            that wrote them).  Elements must be finite.
 *   src    : IL_SRC_F32 or IL_SRC_BF16.
 *   fmt    : IL_Q8 or IL_Q4 (IL_BF16 is rejected: nothing to quantise to).
 *   n_out, n_in : as for il_upload (n_in a positive multiple of 32).
 * The handle is the same kind il_upload returns: il_download of it yields
 * the host-format blocks of the rule above, and il_matmul uses it like any
 * other.  Synchronous.  Returns NULL on failure (bad arguments, no device,
 * out of memory); the reason is in il_last_error(). */
IL_API il_weight *il_upload_quantize(const void *weight, il_src src, il_fmt fmt, int64_t n_out, int64_t n_in);

/* Export -- writes the weight of a handle back in its host format (see
 * il_fmt: bf16 words, or the Q8 / Q4 blocks), bit for bit what il_upload
 * would accept to recreate it.
 *   host_out : HOST buffer of at least il_weight_bytes(w) bytes, or NULL.
 *   cap      : size of host_out in bytes.
 * Returns the number of bytes the host format needs; the bytes are written
 * only when host_out is not NULL and cap is at least that number (so a call
 * with NULL, 0 is a size query).  Synchronous.  Returns -1 on failure (NULL
 * handle, device error), with the reason in il_last_error(). */
IL_API int64_t il_download(const il_weight *w, void *host_out, int64_t cap);

/* Drops a handle and its device memory.  NULL is ignored.  The caller must
 * make sure no il_matmul still using it is in flight (synchronize the
 * streams it was used on first). */
IL_API void il_free(il_weight *w);

/* Backend::matmul -- run every job over the shared x in one submission.
 *   x       : DEVICE pointer to float[t][n_in] row-major, 16-byte aligned.
 *   t       : rows of x (tokens); t == 0 or n_jobs == 0 is a no-op.
 *   n_in    : columns of x; must match every job's weight.
 *   jobs    : HOST array of n_jobs job descriptors (read during the call).
 *   hip_stream : hipStream_t to enqueue on (NULL = the null stream).
 * Validates every job first; any invalid job fails the whole call before
 * anything is enqueued (all or nothing).  Paths by t: t <= 8 the decode
 * GEMV kernels (f32 streaming or matrix-core, by format and t), one launch
 * per weight format present; 8 < t <= 32 the matrix-core kernel's wide
 * mode; beyond, the MFMA GEMM: an x -> bf16 pre-pass, then one launch per
 * format (bf16: whole rounds of 256 x 256 tiles and the rest as 128 x 128
 * quarters; Q8/Q4: 256 x 128 halves and 128 x 128 quarters, the codes exact
 * and each block's scale applied to its f32 partial sum; Q8/Q4 with
 * t <= 128: units holding every token, whose last partial round is split
 * over K and completed by a third, small launch).  All jobs of one format
 * share each launch.  Accuracy: every y element is within 4e-3 of the sum
 * of |x_k * w_k| over its reduction of the exact result; the f32 streaming
 * decode kernel keeps x in f32, the matrix-core paths (decode, wide mode
 * and GEMM) round x to bf16 (nearest even, < 3.9e-3 relative) and nothing
 * else: codes, scales and products are exact, sums in f32.  The bf16 copy of x (and the split units' partial
 * sums) live in a buffer the library keeps per stream (grown when a call
 * needs more, kept until the process ends; while the stream is being
 * captured into a graph and that buffer is too small, the call allocates
 * stream-ordered memory instead).  A graph that captured a prefill call
 * reads the buffer of the stream it was captured on: do not replay it
 * concurrently with other prefill calls on that stream.  Asynchronous:
 * returns after enqueueing, results are valid once the stream has reached
 * that point.
 * Returns 1 on success, 0 if nothing was computed (the page's `false`: the
 * caller then runs the whole batch elsewhere).  On a validation failure the
 * y buffers are untouched; if a launch itself fails their contents are
 * unspecified.  The reason is in il_last_error(). */
IL_API int il_matmul(const float *x, int64_t t, int64_t n_in, const il_job *jobs, int64_t n_jobs,
              void *hip_stream);

/* il_matmul for callers that cannot allocate device memory: code being
 * captured into a HIP graph that must hold no allocation nodes, serving loops
 * that may not call hipMalloc, harnesses that forbid it.  Same arguments,
 * validation, kernels, results and 1 / 0 return as il_matmul, but the call
 * allocates nothing (no device memory, no events): the bf16 copy of x that
 * the prefill path (t > 8) reads, and the partial sums of units split over
 * K, live in a static buffer of 32 MiB per device, built into the library
 * and held until the process ends.
 *   - Limit: a prefill call needs t * n_in * 2 bytes (rounded up to 256) for
 *     that copy, plus, for Q8/Q4 at 32 < t <= 128, 8 MiB (t <= 64) or
 *     16 MiB of partial sums and 256 bytes; when that exceeds 32 MiB (bf16
 *     weights: t * n_in > 16777216) the call fails before enqueueing
 *     anything, y untouched, with the sizes in il_last_error().  Decode
 *     calls (t <= 8) and the mid-size calls that round x themselves
 *     (t <= 16) use no scratch.
 *   - Every call on a device shares that device's buffer: calls that overlap
 *     on one device (from several streams, or a replayed graph next to other
 *     work) race on it; order them on one stream or synchronize between them.
 *   - The first call on a device looks up the buffer's address (no
 *     allocation); the device must be current, as for il_matmul. */
IL_API int il_matmul_noalloc(const float *x, int64_t t, int64_t n_in, const il_job *jobs, int64_t n_jobs,
                             void *hip_stream);

/* Fused feed-forward gate/up step -- in one submission,
 *     y[t][n_out] = GELU(x * G^T) (.) (x * U^T)        (element-wise product)
 * the `matmul_multi` over the gate and up projections followed by
 * `gelu_mul(&mut g, &u)` in `Drafter::step` on the oxinfer 0.0.1
 * src/drafter.rs page, without writing g or u to memory.  The page does not
 * print gelu_mul; GELU here is the plain definition
 *     GELU(v) = v * Phi(v) = 0.5 * v * (1 + erf(v / sqrt(2))).
 *   x        : DEVICE float[t][n_in], 16-byte aligned (as for il_matmul).
 *   gate, up : handles of the same format with shape [n_out, n_in].
 *   y        : DEVICE float[t][n_out] row-major, written in full; must not
 *              overlap x.
 *   hip_stream : as for il_matmul.
 * Accuracy: g and u are formed by the same kernels as il_matmul, so y is
 * within the propagation of their tolerance through GELU (slope <= 1.13).
 * Validation, stream semantics and the 1 / 0 return follow il_matmul;
 * t == 0 is a no-op. */
IL_API int il_matmul_gelu_mul(const float *x, int64_t t, int64_t n_in, const il_weight *gate,
                              const il_weight *up, int64_t n_out, float *y, void *hip_stream);

/* Centroid-masked LM head -- for each row x of a batch, the argmax token
 * over a centroid-selected subset of the vocabulary (the end of
 * `Drafter::step` on the oxinfer 0.0.1 src/drafter.rs page):
 *   1. centroid logits cl[c] = centroids[c] . x (c < C);
 *   2. the top_k centroids of largest logit, visited by decreasing logit and,
 *      among equal logits, increasing index (the page's select_nth_unstable
 *      leaves this order open; this is the reading taken);
 *   3. the score embed[tok] . x of every token tok = ordering[c * V/C + j]
 *      (j < V/C) of those clusters, and the first token of largest score met
 *      in visiting order (clusters in step-2 order, tokens in j order).
 * Logits and scores are f32 sums of bf16 x f32 products; where two logits or
 * scores are closer than their rounding, either choice is correct.
 *   x          : DEVICE float[t][h], 16-byte aligned; 1 <= t <= 8.
 *   centroids  : bf16 handle [C, h];  embed : bf16 handle [V, h], V % C == 0.
 *   ordering   : DEVICE uint32[V]; entries >= V are skipped (never chosen).
 *   top_k      : >= 1; a value above C means every cluster (k = min(top_k,
 *                C), as the page's `top_k_centroids.min(num_centroids)`);
 *                (C + h + 2 * next_pow2(k)) * 4 bytes must fit in 152 KiB
 *                (one workgroup's LDS less 8 KiB).
 *   token      : DEVICE int32[t]: the chosen token (-1 if every candidate of
 *                the row was skipped).
 *   clusters   : DEVICE int32[t][k] or NULL: the chosen clusters in
 *                visiting order (k = min(top_k, C)).
 *   score      : DEVICE float[t] or NULL: the chosen token's score.
 *   workspace  : DEVICE scratch of at least il_centroid_argmax_workspace(t,
 *                C, top_k) bytes, owned by the caller and not used by
 *                anything else until the stream has passed this call; or
 *                NULL, and the library allocates it stream-ordered (slower:
 *                allocation nodes in graphs, ~15 us per call measured).
 *   hip_stream : as for il_matmul.
 * Validation, stream semantics and the 1 / 0 return follow il_matmul. */
IL_API int il_centroid_argmax(const float *x, int64_t t, int64_t h, const il_weight *centroids,
                              const il_weight *embed, const uint32_t *ordering, int64_t top_k, int32_t *token,
                              int32_t *clusters, float *score, void *workspace, int64_t workspace_bytes,
                              void *hip_stream);

/* Bytes of workspace il_centroid_argmax needs for t rows, C centroids and
 * top_k clusters (t * (C + 2 * k) * 4 with k = min(top_k, C)); -1 for sizes
 * it does not take. */
IL_API int64_t il_centroid_argmax_workspace(int64_t t, int64_t n_centroids, int64_t top_k);

/* Backend::wants -- whether a matmul of these dimensions is worth running on
 * the GPU (the page: dispatch has a fixed cost, so small ops stay on the
 * CPU).  A pure function of the sizes: 1 if 2 * n_out * n_in * t is at least
 * the threshold (default 2^18 flops, IL_WANTS_MIN_FLOP in the environment
 * overrides it), else 0.  Advisory only: il_matmul never consults it. */
IL_API int il_wants(int64_t n_out, int64_t n_in, int64_t t);

/* Measurement aid, not part of the layer: a plain streaming read of
 * `bytes` bytes of device memory with no arithmetic beside the loads -- the
 * ceiling the decode kernels' weight bandwidth (the GB/s of
 * `WeightRef::bytes`) is compared with.
 *   buf        : DEVICE pointer, `bytes` readable bytes (bytes >= 1).
 *   chunk      : bytes per workgroup, a multiple of 16 in [1024, 2^31);
 *                ceil(bytes / chunk) workgroups.
 *   waves      : waves per workgroup, 1..16.
 *   depth      : 16-byte loads in flight per lane: 1, 2, 4, 8 or 16.
 *   sink       : DEVICE buffer of at least 4 * ceil(bytes / chunk) bytes
 *                (sink_bytes); one word per workgroup is written (an XOR of
 *                the words it read), so the loads cannot be optimised away.
 *   hip_stream : as for il_matmul.
 * Asynchronous; returns 1 after enqueueing, 0 on bad arguments (reason in
 * il_last_error()). */
IL_API int il_read_probe(const void *buf, int64_t bytes, int64_t chunk, int waves, int depth, void *sink,
                         int64_t sink_bytes, void *hip_stream);

/* Backend::name -- a static string naming this backend. */
IL_API const char *il_name(void);

/* Backend::stats -- cumulative summary (calls, jobs and weight bytes per
 * kernel path -- decode GEMV, prefill GEMM, upload quantiser, whose bytes are
 * the full-precision input; device times of the kernels, from HIP events
 * around their launches, when IL_TIMING=1 is set) written as text into
 * buf (NUL-terminated, truncated to cap bytes).  Returns the length the full
 * text needs, excluding the NUL; buf may be NULL when cap is 0. */
IL_API int64_t il_stats(char *buf, int64_t cap);

/* The weight's host-format size in bytes (`WeightRef::bytes`): bf16
 * 2*n_out*n_in, Q8 36*n_out*n_in/32, Q4 18*n_out*n_in/32.  -1 for NULL. */
IL_API int64_t il_weight_bytes(const il_weight *w);

/* Message of the last failure on this thread ("" if none). */
IL_API const char *il_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* IL_H */
