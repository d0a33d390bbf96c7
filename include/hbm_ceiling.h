/*
 * hbm_ceiling — a measured memory ceiling for the Bi-WKV forward's byte mix (measurement only).
 *
 * The Bi-WKV forward of the Vision-RWKV article ("OpenGVLab&港中文&复旦&南大&清华提出Vision-RWKV
 * Backbone", section "Linear Complexity Bidirectional Attention", Eq. (5)) is bound by HBM: it
 * reads k and v once and writes one fp32 output per element. hbm_stream moves exactly those
 * bytes with out = k + v and no other work, so its duration is the time this device needs for
 * that byte mix. It is not part of the Bi-WKV computation.
 */
#ifndef LIBBIWKV_HBM_CEILING_H
#define LIBBIWKV_HBM_CEILING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HBM_F32 0
#define HBM_BF16 1

#define HBM_OK 0
#define HBM_ERR_ARG (-1) /* bad dtype, mode, unroll, policy, size, NULL or misaligned pointer */
#define HBM_ERR_HIP (-2) /* the launch failed */

/*
 * Streams n elements: mode 0 reads k and v (dtype HBM_BF16 or HBM_F32, [n]) and writes
 * out[i] = k[i] + v[i] (fp32, [n]); mode 1 only reads k and v; mode 2 only writes out.
 *   k, v, out : device pointers, 16-byte aligned; the caller owns them; out must not overlap.
 *   n         : a multiple of 8 (bf16) or 4 (fp32); with policy bit 2, of 4 (bf16) or 2 (fp32).
 *   blocks    : 256-thread workgroups of the grid-stride loop (0: one piece per thread).
 *   unroll    : 1, 2, 4 or 8 pieces per thread per loop trip, all loads issued before any store.
 *   policy    : bit 0 non-temporal loads, bit 1 non-temporal stores, bit 2 8-byte pieces of k
 *               and v per thread (4 bf16 or 2 fp32 elements) instead of 16-byte ones.
 *   stream    : hipStream_t as void* (NULL: the null stream). Asynchronous; nothing allocated.
 * Returns HBM_OK, HBM_ERR_ARG (nothing launched) or HBM_ERR_HIP.
 */
int hbm_stream(const void* k, const void* v, float* out, int64_t n, int dtype, int mode, int blocks,
               int unroll, int policy, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBBIWKV_HBM_CEILING_H */
