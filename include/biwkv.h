/*
 * libbiwkv — Vision-RWKV spatial-mix hot path for AMD Instinct MI355X (gfx950).
 *
 * Operations (cited by page title and equation; the pages define what is computed):
 *   Bi-WKV   — "OpenGVLab&港中文&复旦&南大&清华提出Vision-RWKV Backbone" (Vision-RWKV article),
 *              section "Linear Complexity Bidirectional Attention", Eq. (5) (summation form) and
 *              Eq. (6)-(7) (the four-state RNN form the library evaluates as a chunked scan):
 *                wkv_t = ( sum_{i != t} e^{-((|t-i|-1)/T) w + k_i} v_i + e^{u + k_t} v_t )
 *                      / ( sum_{i != t} e^{-((|t-i|-1)/T) w + k_i}     + e^{u + k_t}     )
 *              per batch item and channel; w (decay, any sign) and u (bonus) are per-channel.
 *              The exponent is divided by T as the article's "Scale Up Stability" section asks.
 *   Q-Shift  — the q_shift function in "LinXin's Blog" Vision-RWKV notes (and Eq. (9) of the
 *              article, whose direction order the listing supersedes): on the H x W token grid
 *              (token n = h*W + w), channel groups [0,g1) shift right, [g1,g2) left, [g2,g3) down,
 *              [g3,g4) up by `shift` tokens with zero fill; channels >= g4 are copied;
 *              g_j = int(C * gamma * j) computed in double precision as in the listing.
 *   Fused    — Bi-WKV applied to Q-Shift(k) and Q-Shift(v), with T = H*W. Zero-filled sources
 *              enter the attention as k = 0, v = 0 (they are values, not masks).
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers of the current HIP device, except where stated. Arrays are
 *     contiguous; [B, T, C] means C is the fastest-varying index.
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream. Calls are asynchronous:
 *     they validate on the host, enqueue, and return. No call synchronises.
 *   - The caller owns every buffer. The library keeps no pointer to caller memory after the
 *     enqueued work completes. Bi-WKV calls whose sequence is split over several workgroups
 *     (fp32: T above 512; bf16: T above 1024, or above 512 when B * ceil(C / 64) exceeds the
 *     device's compute units) use library-owned scratch (chunk sums and a small counter block)
 *     kept per (device, stream); it is allocated in stream order
 *     (hipMallocAsync) on the first such call on a stream, grown when a larger problem arrives
 *     (the outgrown buffer is freed in stream order), and released by biwkv_release_scratch. So
 *     those calls must not be made under HIP graph capture unless an earlier call on the stream
 *     already sized the scratch. Replaying a captured call is safe: launches are told apart by a
 *     device-side epoch, not by arguments.
 *   - A row split over several workgroups is combined either in one launch, where the chunks of
 *     a row exchange their sums while resident (used when every workgroup of the launch fits on
 *     the device at once, or when a row's chunks take at most a quarter of the workgroups that
 *     fit: later rows then start as earlier ones finish), or in the two-pass form: 128-token
 *     chunks' sums, a per-row scan of them into each chunk's carries, then the outputs (three
 *     launches, nothing waits). In one launch a workgroup waits a bounded time for a peer chunk's
 *     sums and then recomputes them from that chunk's k and v, so results never depend on the
 *     peers being resident (for example when other work occupies the device);
 *     biwkv_stream_fault_flags reports that this happened.
 *   - All argument validation happens on the host before any HIP call. A problem with zero
 *     elements returns BIWKV_OK without enqueuing anything. Nothing is printed; no C++ exception
 *     crosses this interface.
 *   - Thread safety: calls may come from several host threads. Calls on the same stream are
 *     serialised by the stream; calls on different streams use different scratch.
 */
#ifndef LIBBIWKV_BIWKV_H
#define LIBBIWKV_BIWKV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type of k and v. Bi-WKV always accumulates and writes in fp32. */
#define BIWKV_F32 0   /* IEEE binary32 */
#define BIWKV_BF16 1  /* bfloat16 (upper half of a binary32) */

/* Status codes. */
#define BIWKV_OK 0
#define BIWKV_ERR_NULL (-1)        /* a required pointer is NULL                                 */
#define BIWKV_ERR_SHAPE (-2)       /* a dimension < 0, too large, or T != H*W                    */
#define BIWKV_ERR_DTYPE (-3)       /* dtype is neither BIWKV_F32 nor BIWKV_BF16                  */
#define BIWKV_ERR_PARAM (-4)       /* gamma outside [0, 1/4] or NaN; shift < 0 or > min(H, W)   */
#define BIWKV_ERR_ALIAS (-5)       /* out overlaps an input                                      */
#define BIWKV_ERR_ALIGN (-6)       /* a pointer is not aligned to its element size               */
#define BIWKV_ERR_NO_DEVICE (-7)   /* no usable HIP device                                       */
#define BIWKV_ERR_HIP (-8)         /* a HIP runtime call or launch failed; see biwkv_last_hip_error */
#define BIWKV_ERR_UNSUPPORTED (-9) /* a shape outside the kernels' addressing (limits per entry)  */
#define BIWKV_ERR_SCRATCH (-10)    /* biwkv_forward_noalloc: chunk sums beyond its static buffer */

/* Options (biwkv_set_option). Process-wide; they apply to calls made after they are set. */
#define BIWKV_OPT_SPIN_LIMIT 1 /* polls of a peer chunk's sums before recomputing them (default 4096;
                                  0: recompute every peer's sums without waiting; the backward
                                  then hands every row of several chunks to its fallback)    */
#define BIWKV_OPT_TWO_PASS 2   /* 0 (default): one launch when all workgroups fit at once or
                                  a row's chunks take at most a quarter of the resident
                                  workgroups; 1: every row takes the two-pass form (the
                                  backward: its multi-launch form); 2: one launch whenever a
                                  row's chunks fit at once (forward entries)                  */
#define BIWKV_OPT_WIDE_INDEX 3 /* 0 (default): Q-Shift gathers use 32-bit index arithmetic below
                                  2^31 items; 1: always the 64-bit form                       */
#define BIWKV_OPT_XCD_LOCAL 4  /* 1 (default): a one-launch row (forward or backward) runs all
                                  its chunks on one XCD and exchanges their sums through that
                                  XCD's L2; 0: plain block order, sums through the
                                  device-coherent level                                       */

/*
 * Bi-WKV forward, Eq. (5) of the Vision-RWKV article.
 *   k, v : [B, T, C], storage type `dtype` (BIWKV_F32 or BIWKV_BF16), device memory.
 *   w, u : [C] float32, device memory (decay, divided by T inside; bonus).
 *   out  : [B, T, C] float32, device memory; must not overlap k, v, w or u.
 * Errors: BIWKV_ERR_NULL, _SHAPE (B, T, C < 0 or B*T*C*4 bytes overflow), _DTYPE, _ALIAS, _ALIGN,
 * _NO_DEVICE, _HIP, and _UNSUPPORTED when one chunk of a row spans 2^31 bytes of out: a chunk is
 * the whole row only while B * ceil(C / 64) is at most the device's compute units (so C is small),
 * and at most 512 tokens otherwise, so C * 512 * 4 must stay below 2^31 (C < 1048576). Any T up
 * to 2^31 - 1 is addressed.
 */
int biwkv_forward(const void* k, const void* v, const float* w, const float* u, float* out,
                  int64_t B, int64_t T, int64_t C, int dtype, void* stream);

/*
 * Allocation-free Bi-WKV forward, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the same computation,
 * arguments, layout and errors as biwkv_forward, with the same kernels, but the scratch of rows
 * split over several workgroups lives in a static device array of the library (256 bytes of
 * counters and 8 MiB of chunk sums per device, held until the process ends) instead of
 * per-stream buffers. The call allocates nothing: no hipMalloc, hipFree or allocating library
 * routine (the array's address is looked up once per device, on the first call there). Every
 * call on a device shares that array, and it keeps the last call's contents: calls that overlap
 * on one device (several streams or threads at once) race and must not be made. A row of several
 * chunks needs 3 KiB per chunk in one launch (B * ceil(C / 64) * ceil(T / 512) chunks of 512
 * tokens in general; bf16 rows of up to 896 tokens split into chunks of 448) and 4 KiB per
 * 128-token chunk in the two-pass form; a problem that needs more than 8 MiB returns
 * BIWKV_ERR_SCRATCH before anything is enqueued.
 */
int biwkv_forward_noalloc(const void* k, const void* v, const float* w, const float* u, float* out,
                          int64_t B, int64_t T, int64_t C, int dtype, void* stream);

/*
 * Bi-WKV backward: gradients of a loss L through out = Bi-WKV(k, v) (Eq. (5) of the Vision-RWKV
 * article; the article states an O(TC) backward recurrence without printing it, and the
 * gradients here follow from Eq. (5)). Given g = dL/dout:
 *   dk, dv : [B, T, C] float32, device memory (dL/dk, dL/dv; written, not accumulated).
 *   dw, du : [C] float32, device memory (dL/dw, dL/du summed over the batch; written).
 *   k, v, w, u, B, T, C, dtype: as for biwkv_forward; g: [B, T, C] float32, device memory.
 * Outputs must not overlap each other or any input. The pass recomputes the forward sums, so it
 * needs no forward state. Launch forms:
 *  - a row of up to 64 tokens: one launch, no scratch but the dw / du terms;
 *  - a longer row whose 128-token chunks take at most a quarter of the workgroups resident on the
 *    device (B * ceil(C / 64) rows of ceil(T / 128) chunks; T up to 16384 on MI355X): one launch
 *    in which the chunks of a row exchange both rounds' sums while they run (96 bytes per chunk
 *    and tile channel of tagged sums), then one more kernel for dw and du. A workgroup whose
 *    bounded wait for a peer runs out (BIWKV_OPT_SPIN_LIMIT) stores nothing and marks its row;
 *    that last kernel then computes every marked row again with one workgroup that needs no
 *    other, so no result depends on the chunks being resident together, and
 *    biwkv_stream_fault_flags reports that it happened;
 *  - otherwise (or with BIWKV_OPT_TWO_PASS = 1) five launches that pass per-chunk sums and carries
 *    (64-token chunks) from one to the next.
 * Scratch is library-owned per (device, stream): the tagged sums, and 4 * (2 * B * n * C +
 * 4 * 384 * B * ceil(C / 64) * n) bytes of dw / du terms and chunk sums (n chunks per row),
 * allocated on the first call and grown when a larger problem arrives (so the first call on a
 * stream must not be made under graph capture). dw and du are folded in a fixed order: results
 * are bitwise reproducible. With B * T == 0 (and C > 0), dw and du are set to 0.
 * Errors: BIWKV_ERR_NULL, _SHAPE, _DTYPE, _ALIAS, _ALIGN, _NO_DEVICE, _HIP, and _UNSUPPORTED for
 * T >= 2^24 (token positions must be exact in fp32) or (T + 64) * C * 4 >= 2^31 (one batch item
 * of g is addressed with 32-bit byte offsets).
 */
int biwkv_backward(const void* k, const void* v, const float* w, const float* u, const float* g,
                   float* dk, float* dv, float* dw, float* du, int64_t B, int64_t T, int64_t C,
                   int dtype, void* stream);

/*
 * Causal attention: the original RWKV attention that the Vision-RWKV article (section "Linear
 * Complexity Bidirectional Attention") extends to both directions, i.e. Eq. (7) without the
 * backward states b and d:
 *   out_t = ( sum_{i<t} e^{-((t-1-i)/T) w + k_i} v_i + e^{u+k_t} v_t )
 *         / ( sum_{i<t} e^{-((t-1-i)/T) w + k_i}     + e^{u+k_t}     )
 * w is divided by T as in Eq. (5); the original, undivided decay w0 is w = T * w0.
 * Arguments, layout, ownership, scratch and errors are those of biwkv_forward.
 */
int biwkv_causal_forward(const void* k, const void* v, const float* w, const float* u, float* out,
                         int64_t B, int64_t T, int64_t C, int dtype, void* stream);

/*
 * Gated Bi-WKV, the spatial-mix output of Eq. (2) of the Vision-RWKV article before its output
 * projection: out = sigmoid(r) * Bi-WKV(k, v), elementwise, with sigmoid(x) = 1 / (1 + e^{-x}).
 *   r : [B, T, C] gate input (the R projection), storage type `dtype` like k and v, device memory;
 *       must not overlap out.
 * Other arguments, layout, ownership, scratch and errors are those of biwkv_forward.
 */
int biwkv_gated_forward(const void* k, const void* v, const void* r, const float* w, const float* u,
                        float* out, int64_t B, int64_t T, int64_t C, int dtype, void* stream);

/*
 * Q-Shift token shift X-dagger of the q_shift listing (LinXin's Blog, Vision-RWKV notes).
 *   x, out : [B, H*W, C] float32, device memory; values are moved bit for bit (NaN payloads,
 *            signed zeros and denormals are preserved); out must not overlap x.
 *   shift  : grid offset in tokens, 0 <= shift <= min(H, W).
 *   gamma  : channel-group fraction, 0 <= gamma <= 1/4 (the listing asserts gamma <= 1/4).
 * Errors: BIWKV_ERR_NULL, _SHAPE, _PARAM, _ALIAS, _ALIGN, _NO_DEVICE, _HIP.
 */
int qshift(const float* x, float* out, int64_t B, int64_t H, int64_t W, int64_t C, int shift,
           double gamma, void* stream);

/*
 * Q-Shift mixing, Eq. (9) of the Vision-RWKV article ("Quad-Directional Token Shift") as printed,
 * once per mixing vector: out[j] = x + (1 - mu[j]) * X-dagger(x), j = 0 .. n_mix-1 (e.g. the R, K
 * and V inputs of the spatial-mix projections), with X-dagger the gather of `qshift`.
 *   x   : [B, H*W, C] float32, device memory.
 *   mu  : [n_mix, C] float32, device memory.
 *   out : [n_mix, B, H*W, C] float32, device memory; must not overlap x or mu.
 *   n_mix : 0 .. 8. shift, gamma: as for qshift.
 * fp32 arithmetic x + (1 - mu) * xd per element (the compiler may fuse the multiply-add).
 * Errors: as qshift, plus _SHAPE for n_mix outside 0 .. 8.
 */
int qshift_mix(const float* x, const float* mu, float* out, int64_t B, int64_t H, int64_t W,
               int64_t C, int n_mix, int shift, double gamma, void* stream);

/*
 * Fused Q-Shift + Bi-WKV: out = Bi-WKV(Q-Shift(k), Q-Shift(v)) with T = H*W. The shift is applied
 * while k and v are loaded; no shifted copy is written to memory.
 *   k, v : [B, H*W, C], storage type `dtype`; w, u : [C] float32; out : [B, H*W, C] float32.
 *   shift, gamma as for qshift().
 * Errors: as biwkv_forward() plus BIWKV_ERR_PARAM; _UNSUPPORTED when (512 + 2 shift W) * C * 4
 * reaches 2^31 (a chunk's loads reach s W tokens on either side).
 */
int biwkv_qshift_forward(const void* k, const void* v, const float* w, const float* u, float* out,
                         int64_t B, int64_t H, int64_t W, int64_t C, int shift, double gamma,
                         int dtype, void* stream);

/*
 * Bidirectional token shift for sparse inputs: the form of Q-Shift that the MAE pre-training
 * paragraph of the Vision-RWKV article uses when only the visible tokens of a masked image are
 * present (there is no H x W grid). The channel groups of qshift keep the sense of their move
 * along the token sequence: channels [0, g1) and [g2, g3) (moved right and down by qshift) take
 * token n - shift, channels [g1, g2) and [g3, g4) (left and up) take token n + shift, with zero
 * fill past either end; channels >= g4 are copied. g_j = int(C * gamma * j) as for qshift.
 *   x, out : [B, N, C] float32, device memory; bit copies; out must not overlap x.
 *   shift  : 0 <= shift <= N.  gamma: 0 <= gamma <= 1/4.
 * Errors: BIWKV_ERR_NULL, _SHAPE, _PARAM, _ALIAS, _ALIGN, _NO_DEVICE, _HIP.
 */
int qshift_bidir(const float* x, float* out, int64_t B, int64_t N, int64_t C, int shift,
                 double gamma, void* stream);

/*
 * Fused bidirectional shift + Bi-WKV: out = Bi-WKV(qshift_bidir(k), qshift_bidir(v)) with T = N
 * (the spatial mix of a sparse, MAE-masked input). The shift is applied while k and v are loaded.
 *   k, v : [B, N, C], storage type `dtype`; w, u : [C] float32; out : [B, N, C] float32.
 *   shift, gamma as for qshift_bidir().
 * Errors: as biwkv_forward() plus BIWKV_ERR_PARAM; _UNSUPPORTED when (512 + 2 shift) * C * 4
 * reaches 2^31.
 */
int biwkv_qshift_bidir_forward(const void* k, const void* v, const float* w, const float* u,
                               float* out, int64_t B, int64_t N, int64_t C, int shift, double gamma,
                               int dtype, void* stream);

/* Static, NUL-terminated description of a status code. Never NULL. */
const char* biwkv_status_string(int status);

/* Raw hipError_t value of the most recent BIWKV_ERR_HIP returned on the calling host thread. */
int biwkv_last_hip_error(void);

/*
 * Diagnostic: synchronises `stream`, then reports and clears the device-side fault word of that
 * stream's scratch. *flags receives 0 when every single-launch Bi-WKV call on the stream since
 * the last query found its peer chunks' sums published in time; bit 0 set means that at least one
 * workgroup's bounded wait ran out and it recomputed a peer chunk's sums from k and v (the outputs
 * are still correct: this is a slow path, not an error). Returns BIWKV_OK, BIWKV_ERR_NULL (flags
 * NULL), _NO_DEVICE or _HIP. A stream with no scratch yet reports 0.
 */
int biwkv_stream_fault_flags(void* stream, uint32_t* flags);

/*
 * Releases the library's scratch for (current device, `stream`) in stream order: the memory is
 * freed once the work already queued on the stream is done. Call it before destroying a stream
 * that made Bi-WKV calls; a later call on the stream allocates fresh scratch. Returns BIWKV_OK
 * (also when the stream has no scratch), _NO_DEVICE or _HIP.
 */
int biwkv_release_scratch(void* stream);

/*
 * Sets process-wide option `option` (BIWKV_OPT_*) to `value`; the previous value is written to
 * *previous unless it is NULL. BIWKV_OPT_SPIN_LIMIT takes 0 .. 2^32 - 1, BIWKV_OPT_TWO_PASS 0, 1
 * or 2, the others 0 or 1.
 * Calls already enqueued are not affected. Returns BIWKV_OK or BIWKV_ERR_PARAM (unknown option or
 * value out of range; nothing changed).
 */
int biwkv_set_option(int option, int64_t value, int64_t* previous);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int biwkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBBIWKV_BIWKV_H */
