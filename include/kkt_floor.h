/* Memory-traffic reference for the fused chunk-local KKT + solve.
 *
 * Not part of the operation: a kernel that moves exactly the bytes one call
 * of kkt_solve moves on sequences of whole 64-token chunks (the key rows, g
 * and beta in; the output rows out), in the fused kernel's access pattern
 * (one chunk of one head per wave, all of a wave's loads before its stores,
 * non-temporal whole-row stores, launch arguments preloaded into SGPRs),
 * with no arithmetic.  Its time bounds from
 * below what a kernel with this data movement takes on the machine; the
 * benchmark reports it beside the fused op (bench.py --op floor).
 *
 * Built as libkkt_floor.so, separate from libkkt_solve.so.
 */
#ifndef KKT_FLOOR_H
#define KKT_FLOOR_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Copies key rows to output rows on `stream` (NULL: the default stream).
 *   k:    [B, T, H] rows of key_row_bytes bytes, contiguous, device memory
 *   g, beta: [B, T, H] fp32, device memory, or NULL (then not read)
 *   out:  [B, T, H] rows of out_row_bytes bytes, contiguous, device memory
 * Output: 16-byte piece c of output row (b, t, h) holds piece
 * c mod (key_row_bytes / 16) of key row (b, t, h).
 * Sizes: B, H >= 1; T a positive multiple of 64 below 2^31; key_row_bytes 128, 256 or
 * 512; out_row_bytes 128 or 256; 64 * H * key_row_bytes and
 * 64 * H * out_row_bytes below 2^31; B * (T / 64) * H below 2^31.
 * Returns 0 when the kernel was launched, 1 for invalid arguments (nothing
 * launched), 2 when the launch failed.  The caller owns every buffer. */
int kkt_floor_copy(const void* k, const float* g, const float* beta, int64_t B, int64_t T, int64_t H,
                   int64_t key_row_bytes, int64_t out_row_bytes, void* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KKT_FLOOR_H */
