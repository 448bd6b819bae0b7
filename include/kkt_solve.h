/*
 * kkt_solve.h: C ABI of the fused chunk-local KKT + triangular solve for
 * AMD Instinct MI355X (gfx950).
 *
 * Operation (MindSpeed-Ops pull request #135, "feat(triton): add
 * chunk_gated_delta_rule_fwd_kkt_solve"; PR description, user-facing-change
 * section and bot change summary):
 *
 *   One call does what the two-step path solve_tril(chunk_scaled_dot_kkt_fwd)
 *   does.  The tokens of every (batch row or sequence, head) are cut into
 *   chunks of 64, restarting at every sequence start; the last chunk of a
 *   sequence may be shorter (L < 64).  For a chunk starting at token t0 with
 *   local rows i, j in [0, L):
 *
 *     A[i][j] = beta_i * (k_i . k_j) * exp(clamp(g_i - g_j, -50, 50))  for i > j
 *     A[i][j] = 0                                                        otherwise
 *
 *     out[b][t0 + i][h][j] = ((I + A)^{-1})[i][j]   for j < L
 *     out[b][t0 + i][h][j] = 0                      for L <= j < 64
 *
 *   so every output row holds its chunk's row of the unit lower-triangular
 *   inverse: 1.0 on the diagonal, +0.0 above it, written in full by the call
 *   (no pre-zeroed output is needed).
 *
 * Threading: every entry point is thread-safe; the library keeps no state
 * besides a per-thread error string, a per-device architecture cache and the
 * two process-wide options of kkt_set_option.
 */
#ifndef KKT_SOLVE_H
#define KKT_SOLVE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  fp32 is IEEE binary32, bf16 is bfloat16, f16 is IEEE binary16. */
typedef enum {
    KKT_DTYPE_F32 = 0,
    KKT_DTYPE_BF16 = 1,
    KKT_DTYPE_F16 = 2
} kkt_dtype_t;

typedef enum {
    KKT_OK = 0,
    KKT_ERR_INVALID_ARGUMENT = 1, /* a pointer, size or dtype is invalid; nothing was launched */
    KKT_ERR_UNSUPPORTED = 2,      /* valid request this build does not serve (chunk_size, K, device) */
    KKT_ERR_HIP = 3               /* the HIP runtime reported an error while querying or launching */
} kkt_status_t;

/*
 * kkt_solve: the fused op (PR #135 page: the fused API takes k, g, beta,
 * cu_seqlens, chunk_size and an output dtype and returns (I+A)^{-1} of shape
 * [B,T,H,64]).  chunk_size 64 is the API's value; 128 is also served (the
 * chunk size of the PyPTO GatedDeltaRule case page's tiling, section 3.2):
 * everything above then holds with chunks of 128 tokens and 128-wide output
 * rows, out [B,T,H,128].  Other values are an error.
 *
 *   k          device, [B,T,H,K] of in_dtype, contiguous (H*K elements per token).
 *   g          device, [B,T,H] fp32 chunk-local cumulative log-decay, or NULL
 *              (no gate: every exp factor is 1).  The caller provides g already
 *              summed within each chunk; only differences g_i - g_j inside a
 *              chunk are used.
 *   beta       device, [B,T,H] fp32 row scale, or NULL (beta = 1).
 *   cu_seqlens device, int32 [num_seqs + 1] start offsets of packed sequences,
 *              or NULL for fixed-length rows.  With cu_seqlens, B must be 1;
 *              offsets are expected to start at 0, not decrease and end at T.
 *              The kernel clamps every offset into [0, T], so malformed
 *              offsets cannot make it access memory outside the tensors; rows
 *              not covered by any sequence are then left unwritten.  With the
 *              option KKT_OPTION_VALIDATE_CU_SEQLENS set (kkt_set_option) the
 *              offsets are copied to the host (synchronously) and checked
 *              first.
 *   num_seqs   number of sequences; ignored when cu_seqlens is NULL.
 *   B, T, H, K sizes.  T may be 0 (nothing is launched) and is below 2^32
 *              (KKT_ERR_UNSUPPORTED otherwise).
 *              K is at most 256 and each key row a whole number of 16-byte
 *              pieces: a multiple of 4 for fp32 keys, of 8 for bf16 / f16
 *              keys.  The PR #135 page shows K = 128 only; the rest is this
 *              library's range (KKT_ERR_UNSUPPORTED otherwise).
 *   chunk_size 64 or 128 (the chunk length; also the width of an output row).
 *   in_dtype   element type of k.
 *   out_dtype  element type of out.  bf16 / f16 results are rounded to nearest
 *              even from the fp32 value.
 * Precision: all arithmetic is fp32.  The dot products k_i . k_j accumulate
 * in fp32 on the matrix cores; 16-bit keys multiply exactly, fp32 keys are
 * split into three bf16 parts (exact to 2^-27 relative) whose six leading
 * part products are summed, so every A entry stays within (K + 128) 2^-24 of
 * |beta_i| sum_k |k_ik k_jk| exp(clamp(g_i - g_j)) whatever the key dtype.
 *   out        device, [B,T,H,chunk_size] of out_dtype, contiguous; every element is
 *              written (for varlen: every element of the rows covered by the
 *              sequences).  Must not overlap any input.
 *   stream     HIP stream the kernel is enqueued on (NULL: the null stream);
 *              it must belong to the calling thread's current device, which
 *              is the device checked to be gfx950.
 *
 * Alignment: k and out 16-byte aligned; g, beta and cu_seqlens 4-byte aligned
 * (KKT_ERR_INVALID_ARGUMENT otherwise).  Every device address lies below 2^48,
 * as GPU virtual addresses do on ROCm (KKT_ERR_UNSUPPORTED otherwise): the
 * kernels receive addresses in 48 bits.
 *
 * Launch form (chunk_size 64): grids of up to 256 chunk-head tiles run each
 * tile on two waves, larger grids one tile per wave; both give bit-identical
 * results.  With 16-bit keys and a 16-bit output every grid takes one wave
 * per tile (on small grids it is the faster form for those types; the
 * gate-sum op and the solve of a given A keep the 256 whatever the types).
 * The option KKT_OPTION_SPLIT_MAX_TILES sets one bound for every call
 * instead (0: always one wave per tile).
 *
 * All pointers are owned by the caller; the library allocates nothing and
 * keeps no pointer after the call returns.  The call is asynchronous: it
 * returns once the kernel is enqueued, and faults during execution surface at
 * the caller's next synchronisation.  Argument errors are detected before
 * any HIP call, return KKT_ERR_INVALID_ARGUMENT / KKT_ERR_UNSUPPORTED and
 * launch nothing; kkt_last_error() then describes the problem.
 */
kkt_status_t kkt_solve(const void* k, const float* g, const float* beta,
                       const int32_t* cu_seqlens, int64_t num_seqs,
                       int64_t B, int64_t T, int64_t H, int64_t K,
                       int64_t chunk_size, kkt_dtype_t in_dtype, kkt_dtype_t out_dtype,
                       void* out, hipStream_t stream);

/*
 * kkt_solve_gate_cumsum: kkt_solve fed with the per-token log-decay instead
 * of its chunk-local sum.  The gate g that kkt_solve takes is the running sum
 * of a per-token log-decay a_t, restarted at every chunk (PR #135 page,
 * user-facing-change section: g is the op's gate argument; this library
 * reads it as that chunk-local sum).  Here the kernel forms the sum itself:
 *
 *   g[t0 + i] = a[t0] + a[t0 + 1] + ... + a[t0 + i]     (i < L, fp32)
 *
 * and then computes exactly what kkt_solve computes with that g.
 *
 *   g_decay    device, [B,T,H] fp32 per-token log-decay; must not be NULL.
 *   g_out      device, [B,T,H] fp32, or NULL: receives the summed gate g of
 *              every covered row (the later steps of the forward pass use
 *              it).  It may be the same pointer as g_decay (the sum is then
 *              done in place); it must not overlap any other argument.
 *   The sum is a 6-level tree (a parallel inclusive scan over 64 rows) in
 *   fp32; with chunk_size 128 the second half's scan is added to the first
 *   half's total (7 levels).  Its result differs from a left-to-right sum by
 *   rounding only.  kkt_solve(k, g_out, ...) with the same chunk_size on the
 *   g_out this call wrote gives bit-identical output.  Everything else
 *   (arguments, chunk_size 64 or 128, alignment, errors, launch form) as for
 *   kkt_solve; g_out must be 4-byte aligned.
 */
kkt_status_t kkt_solve_gate_cumsum(const void* k, const float* g_decay, const float* beta,
                                   const int32_t* cu_seqlens, int64_t num_seqs,
                                   int64_t B, int64_t T, int64_t H, int64_t K,
                                   int64_t chunk_size, kkt_dtype_t in_dtype, kkt_dtype_t out_dtype,
                                   void* out, float* g_out, hipStream_t stream);

/*
 * kkt_scaled_dot: the first step of the unfused two-step path on its own
 * (PR #135 page, PR description: the fused op replaces
 * chunk_scaled_dot_kkt_fwd followed by solve_tril; the first of those forms A).
 *
 *   Writes, for every chunk as defined above,
 *     A_out[b][t0 + i][h][j] = A[i][j]   for j < i < L (the formula above)
 *     A_out[b][t0 + i][h][j] = +0.0      for j >= i
 *   in fp32, shape [B,T,H,64], every element of every covered row written.
 *
 *   k, g, beta, cu_seqlens, num_seqs, B, T, H, K, chunk_size, in_dtype, stream:
 *   as for kkt_solve (same alignment rules, same errors), except that
 *   chunk_size must be 64.  A_out: device,
 *   [B,T,H,64] fp32, contiguous, 16-byte aligned, must not overlap any input.
 *   The A it writes is bit-identical to the A that kkt_solve inverts.
 */
kkt_status_t kkt_scaled_dot(const void* k, const float* g, const float* beta,
                            const int32_t* cu_seqlens, int64_t num_seqs,
                            int64_t B, int64_t T, int64_t H, int64_t K,
                            int64_t chunk_size, kkt_dtype_t in_dtype,
                            float* A_out, hipStream_t stream);

/*
 * kkt_solve_tril: the second step of the unfused path on its own (PR #135
 * page, PR description: solve_tril turns the chunk-local A into (I+A)^{-1}).
 *
 *   A          device, [B,T,H,64] fp32, contiguous, 16-byte aligned.  For every
 *              chunk (cut as above) only the strictly lower entries A[i][j],
 *              j < i < L, are read; the diagonal, the upper part and the
 *              columns j >= L are ignored (they may hold anything).
 *   cu_seqlens, num_seqs, B, T, H, stream: as for kkt_solve; chunk_size must
 *              be 64.
 *   out_dtype, out: as for kkt_solve: rows of (I + strict_lower(A))^{-1},
 *              [B,T,H,64], upper zeros written.  out must not overlap A.
 *
 *   kkt_solve_tril(kkt_scaled_dot(k, ...)) with fp32 A in between gives
 *   bit-identical results to kkt_solve(k, ...): both run the same solve on the
 *   same fp32 values.  Errors and launch form: as for kkt_solve (no K, no
 *   in_dtype here).
 */
kkt_status_t kkt_solve_tril(const float* A, const int32_t* cu_seqlens, int64_t num_seqs,
                            int64_t B, int64_t T, int64_t H, int64_t chunk_size,
                            kkt_dtype_t out_dtype, void* out, hipStream_t stream);

/*
 * Process-wide options.  They change how calls are carried out, never what
 * they compute; they exist for tests and debugging.  A value set takes effect
 * for calls that start after kkt_set_option returns (it is an atomic store;
 * calls already running on other threads may use either value).  Start
 * values are read once, when the library is loaded, from the environment
 * variables named below.
 *
 *   KKT_OPTION_SPLIT_MAX_TILES      grids of up to this many 64-token
 *                                   chunk-head tiles run each tile on two
 *                                   waves (the launch form above); 0: never;
 *                                   -1 (the default; env KKT_SPLIT_TILES):
 *                                   the library's choice, 256 except for
 *                                   kkt_solve with 16-bit keys and output.
 *   KKT_OPTION_VALIDATE_CU_SEQLENS  nonzero: every call with cu_seqlens first
 *                                   copies the offsets to the host
 *                                   (synchronously, on the call's stream) and
 *                                   returns KKT_ERR_INVALID_ARGUMENT unless
 *                                   they start at 0, do not decrease and end
 *                                   at T.  Default 0 (env KKT_VALIDATE=1: on).
 *
 * kkt_set_option returns KKT_ERR_INVALID_ARGUMENT for an unknown option or a
 * KKT_OPTION_SPLIT_MAX_TILES below -1; kkt_get_option returns the current
 * value, or -1 for an unknown option (for KKT_OPTION_SPLIT_MAX_TILES, -1 is
 * also the value that leaves the choice to the library).
 */
typedef enum {
    KKT_OPTION_SPLIT_MAX_TILES = 0,
    KKT_OPTION_VALIDATE_CU_SEQLENS = 1
} kkt_option_t;

kkt_status_t kkt_set_option(kkt_option_t option, int64_t value);
int64_t kkt_get_option(kkt_option_t option);

/* Text of the last non-OK status returned on the calling thread ("" if none).
 * The pointer stays valid until the next kkt_* call on the same thread. */
const char* kkt_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int kkt_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KKT_SOLVE_H */
