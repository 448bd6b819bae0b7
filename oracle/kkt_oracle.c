/*
 * CPU fp64 oracle for the fused chunk-local KKT + triangular solve of the
 * chunked Gated DeltaNet forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * definition that the GPU path is checked against.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it.  It shares no
 * code, header or constant with the HIP library and includes nothing from it.
 *
 * What it computes (sources are the two on-topic web pages):
 *
 *   MindSpeed-Ops pull request #135, "feat(triton): add
 *   chunk_gated_delta_rule_fwd_kkt_solve":
 *     - PR description: one call of the fused op is the same as the two-step
 *       path solve_tril(chunk_scaled_dot_kkt_fwd(...)), i.e. build the
 *       chunk-local gated, beta-scaled K K^T and then solve the unit
 *       lower-triangular system;
 *     - user-facing-change section: signature
 *       (k, g=None, beta=None, cu_seqlens=None, chunk_size=64, output_dtype)
 *       with k of shape [B,T,H,K] and the result (I+A)^{-1} of shape
 *       [B,T,H,64];
 *     - bot change summary: inside a chunk the op forms K @ K^T, does the
 *       lower-triangular solve and outputs the complete (I+A)^{-1}; the gate
 *       exponent is the natural exp of a difference clamped to [-50, 50];
 *       variable-length batches use per-sequence chunk indices and the
 *       sequence's own length for the boundary.
 *
 *   Per chunk of L <= chunk_size rows starting at token t0 (chunks restart at
 *   every sequence boundary), with local indices i, j in [0, L):
 *
 *     A[i][j] = beta_i * (k_i . k_j) * exp(clamp(g_i - g_j, -50, 50))  if i > j
 *     A[i][j] = 0                                                        else
 *     X       = (I + A)^{-1}
 *     out[t0 + i][h][j] = X[i][j]   for j < L,   0 for L <= j < chunk_size
 *
 *   g == NULL means no gate (factor 1); beta == NULL means beta_i = 1.
 *
 * The two steps of the unfused chain are also exposed on their own
 * (kkt_oracle_scaled_dot: A; kkt_oracle_solve_tril: (I + A)^{-1} from A).
 *
 * The gate g the op takes is the chunk-local cumulative log-decay: the running
 * sum, restarted at every chunk, of a per-token log-decay a_t.  The pages use
 * g only in that summed form; kkt_oracle_chunk_cumsum forms it from a_t by
 * that definition (g[t0 + i] = a[t0] + ... + a[t0 + i]), for the entry point
 * that takes a_t itself.
 *
 * The inverse is taken by generic Gauss-Jordan elimination with partial
 * pivoting on the augmented matrix [M | I].  It deliberately does not use the
 * fact that M is unit lower triangular, so that it is an independent route to
 * the forward substitution done on the GPU.
 *
 * Everything is fp64.  Inputs are fp64 copies of the exact input values
 * (bf16, fp16 and fp32 all widen to fp64 without rounding).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KKT_ORACLE_OK 0
#define KKT_ORACLE_BAD_ARGUMENT 1
#define KKT_ORACLE_SINGULAR 2
#define KKT_ORACLE_NO_MEMORY 3

/* Clamp bound of the gate exponent (PR #135 page, bot change summary: the
 * exponent of the gate is clamped to [-50, 50] before exp). */
static const double GATE_CLAMP = 50.0;

/* One chunk: rows t0 .. t0+L-1 of batch b, head h.  Fills A (L x L,
 * row-major, leading dimension L) with the strictly lower gated, beta-scaled
 * Gram matrix defined above. */
static void build_chunk_matrix(const double* k, const double* g, const double* beta,
                               int64_t T, int64_t H, int64_t K, int64_t b, int64_t h,
                               int64_t t0, int64_t L, int clamp_gate, double* A)
{
    for (int64_t i = 0; i < L; ++i) {
        for (int64_t j = 0; j < L; ++j) {
            A[i * L + j] = 0.0;
        }
    }
    for (int64_t i = 0; i < L; ++i) {
        const int64_t ti = (b * T + t0 + i) * H + h; /* index into [B,T,H] */
        const double* ki = k + ti * K;
        for (int64_t j = 0; j < i; ++j) {
            const int64_t tj = (b * T + t0 + j) * H + h;
            const double* kj = k + tj * K;
            double dot = 0.0;
            for (int64_t c = 0; c < K; ++c) {
                dot += ki[c] * kj[c];
            }
            double gate = 1.0;
            if (g != NULL) {
                double d = g[ti] - g[tj];
                if (clamp_gate) {
                    if (d > GATE_CLAMP) d = GATE_CLAMP;
                    if (d < -GATE_CLAMP) d = -GATE_CLAMP;
                }
                gate = exp(d);
            }
            const double b_i = (beta != NULL) ? beta[ti] : 1.0;
            A[i * L + j] = b_i * dot * gate;
        }
    }
}

/* Generic Gauss-Jordan inverse of the n x n matrix M (row-major) with partial
 * pivoting on [M | I].  W is scratch of n * 2n doubles.  Returns 0 on
 * success, nonzero if a zero pivot is met. */
static int gauss_jordan_inverse(int64_t n, const double* M, double* Minv, double* W)
{
    const int64_t w = 2 * n;
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t c = 0; c < n; ++c) {
            W[r * w + c] = M[r * n + c];
            W[r * w + n + c] = (r == c) ? 1.0 : 0.0;
        }
    }
    for (int64_t c = 0; c < n; ++c) {
        /* partial pivoting: the largest magnitude in column c at or below row c */
        int64_t p = c;
        double best = fabs(W[c * w + c]);
        for (int64_t r = c + 1; r < n; ++r) {
            const double v = fabs(W[r * w + c]);
            if (v > best) {
                best = v;
                p = r;
            }
        }
        if (best == 0.0) {
            return 1;
        }
        if (p != c) {
            for (int64_t x = 0; x < w; ++x) {
                const double tmp = W[c * w + x];
                W[c * w + x] = W[p * w + x];
                W[p * w + x] = tmp;
            }
        }
        const double inv_pivot = 1.0 / W[c * w + c];
        for (int64_t x = 0; x < w; ++x) {
            W[c * w + x] *= inv_pivot;
        }
        for (int64_t r = 0; r < n; ++r) {
            if (r == c) continue;
            const double f = W[r * w + c];
            if (f == 0.0) continue;
            for (int64_t x = 0; x < w; ++x) {
                W[r * w + x] -= f * W[c * w + x];
            }
        }
    }
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t c = 0; c < n; ++c) {
            Minv[r * n + c] = W[r * w + n + c];
        }
    }
    return 0;
}

/* Solve one chunk and write its rows of the output. */
static int solve_chunk(const double* k, const double* g, const double* beta,
                       int64_t T, int64_t H, int64_t K, int64_t chunk_size,
                       int64_t b, int64_t h, int64_t t0, int64_t L, int clamp_gate,
                       double* out, double* A, double* M, double* X, double* W)
{
    build_chunk_matrix(k, g, beta, T, H, K, b, h, t0, L, clamp_gate, A);
    for (int64_t i = 0; i < L; ++i) {
        for (int64_t j = 0; j < L; ++j) {
            M[i * L + j] = ((i == j) ? 1.0 : 0.0) + A[i * L + j];
        }
    }
    if (gauss_jordan_inverse(L, M, X, W) != 0) {
        return KKT_ORACLE_SINGULAR;
    }
    for (int64_t i = 0; i < L; ++i) {
        double* row = out + ((b * T + t0 + i) * H + h) * chunk_size;
        for (int64_t j = 0; j < chunk_size; ++j) {
            row[j] = (j < L) ? X[i * L + j] : 0.0;
        }
    }
    return KKT_ORACLE_OK;
}

/* Number of threads the oracle's parallel loop uses. */
int kkt_oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the number of threads of later parallel loops (no effect without OpenMP). */
void kkt_oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* The chunks of a call, in order: batch row or sequence, then position. */
typedef struct {
    int64_t n;
    int64_t* b;
    int64_t* t0;
    int64_t* len;
} chunk_list;

static void free_chunks(chunk_list* c)
{
    free(c->b);
    free(c->t0);
    free(c->len);
}

static int check_and_list_chunks(const int32_t* cu_seqlens, int64_t num_seqs, int64_t B, int64_t T,
                                 int64_t H, int64_t chunk_size, chunk_list* out)
{
    out->n = 0;
    out->b = out->t0 = out->len = NULL;
    if (B < 1 || T < 0 || H < 1 || chunk_size < 1) return KKT_ORACLE_BAD_ARGUMENT;
    if (cu_seqlens != NULL) {
        if (B != 1 || num_seqs < 1 || cu_seqlens[0] != 0 || cu_seqlens[num_seqs] != T) {
            return KKT_ORACLE_BAD_ARGUMENT;
        }
        for (int64_t s = 0; s < num_seqs; ++s) {
            if (cu_seqlens[s + 1] < cu_seqlens[s]) return KKT_ORACLE_BAD_ARGUMENT;
        }
    }
    const int64_t n_rows = (cu_seqlens != NULL) ? num_seqs : B;
    int64_t n_chunks = 0;
    for (int64_t s = 0; s < n_rows; ++s) {
        const int64_t len = (cu_seqlens != NULL) ? (int64_t)cu_seqlens[s + 1] - cu_seqlens[s] : T;
        n_chunks += (len + chunk_size - 1) / chunk_size;
    }
    out->b = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_chunks + 1));
    out->t0 = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_chunks + 1));
    out->len = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_chunks + 1));
    if (out->b == NULL || out->t0 == NULL || out->len == NULL) {
        free_chunks(out);
        return KKT_ORACLE_NO_MEMORY;
    }
    int64_t n = 0;
    for (int64_t s = 0; s < n_rows; ++s) {
        const int64_t bos = (cu_seqlens != NULL) ? cu_seqlens[s] : 0;
        const int64_t eos = (cu_seqlens != NULL) ? cu_seqlens[s + 1] : T;
        for (int64_t t0 = bos; t0 < eos; t0 += chunk_size) {
            out->b[n] = (cu_seqlens != NULL) ? 0 : s;
            out->t0[n] = t0;
            out->len[n] = (eos - t0 < chunk_size) ? (eos - t0) : chunk_size;
            ++n;
        }
    }
    out->n = n;
    return KKT_ORACLE_OK;
}

/*
 * Chunk-local inclusive cumulative sum of a per-token log-decay.
 *   a          [B,T,H] fp64
 *   cu_seqlens, num_seqs, B, T, H, chunk_size: as for kkt_oracle_solve
 *   g_out      [B,T,H] fp64: for every chunk (t0, L) and head h,
 *              g_out[t0 + i][h] = sum_{s=0..i} a[t0 + s][h]   (i < L),
 *              summed left to right in fp64
 * Returns 0, or a nonzero KKT_ORACLE_* code.
 */
int kkt_oracle_chunk_cumsum(const double* a, const int32_t* cu_seqlens, int64_t num_seqs,
                            int64_t B, int64_t T, int64_t H, int64_t chunk_size, double* g_out)
{
    if (a == NULL || g_out == NULL) return KKT_ORACLE_BAD_ARGUMENT;
    chunk_list ch;
    int status = check_and_list_chunks(cu_seqlens, num_seqs, B, T, H, chunk_size, &ch);
    if (status != KKT_ORACLE_OK) return status;
    for (int64_t c = 0; c < ch.n; ++c) {
        for (int64_t h = 0; h < H; ++h) {
            double run = 0.0;
            for (int64_t i = 0; i < ch.len[c]; ++i) {
                const int64_t idx = (ch.b[c] * T + ch.t0[c] + i) * H + h;
                run += a[idx];
                g_out[idx] = run;
            }
        }
    }
    free_chunks(&ch);
    return KKT_ORACLE_OK;
}

/*
 * Full oracle.
 *   k          [B,T,H,K] fp64, contiguous
 *   g, beta    [B,T,H] fp64 or NULL
 *   cu_seqlens [num_seqs+1] int32 sequence offsets or NULL (then every batch
 *              row is one sequence of length T); requires B == 1
 *   out        [B,T,H,chunk_size] fp64, every element written
 *   clamp_gate nonzero: clamp g_i - g_j to [-50, 50] before exp
 * Returns 0, or a nonzero KKT_ORACLE_* code.
 */
int kkt_oracle_solve(const double* k, const double* g, const double* beta,
                     const int32_t* cu_seqlens, int64_t num_seqs,
                     int64_t B, int64_t T, int64_t H, int64_t K,
                     int64_t chunk_size, int clamp_gate, double* out)
{
    if (k == NULL || out == NULL || K < 1) return KKT_ORACLE_BAD_ARGUMENT;
    chunk_list ch;
    int status = check_and_list_chunks(cu_seqlens, num_seqs, B, T, H, chunk_size, &ch);
    if (status != KKT_ORACLE_OK) return status;

    const int64_t n_tiles = ch.n * H;
#pragma omp parallel
    {
        const int64_t cs = chunk_size;
        double* A = (double*)malloc(sizeof(double) * (size_t)(cs * cs));
        double* M = (double*)malloc(sizeof(double) * (size_t)(cs * cs));
        double* X = (double*)malloc(sizeof(double) * (size_t)(cs * cs));
        double* W = (double*)malloc(sizeof(double) * (size_t)(2 * cs * cs));
        int local = (A && M && X && W) ? KKT_ORACLE_OK : KKT_ORACLE_NO_MEMORY;
#pragma omp for schedule(dynamic, 4)
        for (int64_t tile = 0; tile < n_tiles; ++tile) {
            if (local != KKT_ORACLE_OK) continue;
            const int64_t c = tile / H;
            const int64_t h = tile % H;
            const int rc = solve_chunk(k, g, beta, T, H, K, chunk_size, ch.b[c], h,
                                       ch.t0[c], ch.len[c], clamp_gate, out, A, M, X, W);
            if (rc != KKT_ORACLE_OK) local = rc;
        }
        if (local != KKT_ORACLE_OK) {
#pragma omp critical
            status = local;
        }
        free(A);
        free(M);
        free(X);
        free(W);
    }
    free_chunks(&ch);
    return status;
}

/*
 * First step of the unfused chain alone (the pages' chunk_scaled_dot_kkt_fwd,
 * named in the PR #135 description): the strictly lower matrix A of every
 * chunk, row t0+i of A_out holding A[i][0 .. chunk_size-1] (0 for j >= i).
 * Arguments as for kkt_oracle_solve; A_out is [B,T,H,chunk_size] fp64.
 */
int kkt_oracle_scaled_dot(const double* k, const double* g, const double* beta,
                          const int32_t* cu_seqlens, int64_t num_seqs,
                          int64_t B, int64_t T, int64_t H, int64_t K,
                          int64_t chunk_size, int clamp_gate, double* A_out)
{
    if (k == NULL || A_out == NULL || K < 1) return KKT_ORACLE_BAD_ARGUMENT;
    chunk_list ch;
    int status = check_and_list_chunks(cu_seqlens, num_seqs, B, T, H, chunk_size, &ch);
    if (status != KKT_ORACLE_OK) return status;
    const int64_t n_tiles = ch.n * H;
#pragma omp parallel
    {
        const int64_t cs = chunk_size;
        double* A = (double*)malloc(sizeof(double) * (size_t)(cs * cs));
        int local = A ? KKT_ORACLE_OK : KKT_ORACLE_NO_MEMORY;
#pragma omp for schedule(dynamic, 4)
        for (int64_t tile = 0; tile < n_tiles; ++tile) {
            if (local != KKT_ORACLE_OK) continue;
            const int64_t c = tile / H;
            const int64_t h = tile % H;
            const int64_t L = ch.len[c];
            build_chunk_matrix(k, g, beta, T, H, K, ch.b[c], h, ch.t0[c], L, clamp_gate, A);
            for (int64_t i = 0; i < L; ++i) {
                double* row = A_out + ((ch.b[c] * T + ch.t0[c] + i) * H + h) * chunk_size;
                for (int64_t j = 0; j < chunk_size; ++j) row[j] = (j < L) ? A[i * L + j] : 0.0;
            }
        }
        if (local != KKT_ORACLE_OK) {
#pragma omp critical
            status = local;
        }
        free(A);
    }
    free_chunks(&ch);
    return status;
}

/*
 * Second step alone (the pages' solve_tril): reads per chunk the strictly
 * lower part of A (A_in[t0+i][h][j] for j < i; the diagonal and everything
 * above it are ignored) and writes the rows of (I + A)^{-1}, inverted by the
 * same generic Gauss-Jordan elimination.  A_in and out are
 * [B,T,H,chunk_size] fp64.
 */
int kkt_oracle_solve_tril(const double* A_in, const int32_t* cu_seqlens, int64_t num_seqs,
                          int64_t B, int64_t T, int64_t H, int64_t chunk_size, double* out)
{
    if (A_in == NULL || out == NULL) return KKT_ORACLE_BAD_ARGUMENT;
    chunk_list ch;
    int status = check_and_list_chunks(cu_seqlens, num_seqs, B, T, H, chunk_size, &ch);
    if (status != KKT_ORACLE_OK) return status;
    const int64_t n_tiles = ch.n * H;
#pragma omp parallel
    {
        const int64_t cs = chunk_size;
        double* M = (double*)malloc(sizeof(double) * (size_t)(cs * cs));
        double* X = (double*)malloc(sizeof(double) * (size_t)(cs * cs));
        double* W = (double*)malloc(sizeof(double) * (size_t)(2 * cs * cs));
        int local = (M && X && W) ? KKT_ORACLE_OK : KKT_ORACLE_NO_MEMORY;
#pragma omp for schedule(dynamic, 4)
        for (int64_t tile = 0; tile < n_tiles; ++tile) {
            if (local != KKT_ORACLE_OK) continue;
            const int64_t c = tile / H;
            const int64_t h = tile % H;
            const int64_t L = ch.len[c];
            for (int64_t i = 0; i < L; ++i) {
                const double* arow = A_in + ((ch.b[c] * T + ch.t0[c] + i) * H + h) * chunk_size;
                for (int64_t j = 0; j < L; ++j) {
                    M[i * L + j] = (i == j) ? 1.0 : ((j < i) ? arow[j] : 0.0);
                }
            }
            if (gauss_jordan_inverse(L, M, X, W) != 0) {
                local = KKT_ORACLE_SINGULAR;
                continue;
            }
            for (int64_t i = 0; i < L; ++i) {
                double* row = out + ((ch.b[c] * T + ch.t0[c] + i) * H + h) * chunk_size;
                for (int64_t j = 0; j < chunk_size; ++j) row[j] = (j < L) ? X[i * L + j] : 0.0;
            }
        }
        if (local != KKT_ORACLE_OK) {
#pragma omp critical
            status = local;
        }
        free(M);
        free(X);
        free(W);
    }
    free_chunks(&ch);
    return status;
}
