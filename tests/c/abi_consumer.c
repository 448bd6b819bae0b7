/*
 * A plain C consumer of the kkt_solve C ABI (test infrastructure): no Python
 * and no torch, only the HIP runtime for device memory and a stream.
 *
 *   abi_consumer DIR B T H K
 *
 * reads DIR/k.bin (bf16 bit patterns, [B,T,H,K]), DIR/g.bin and DIR/beta.bin
 * (fp32, [B,T,H]), runs on one stream of its own
 *   kkt_solve           -> DIR/x_fused.bin  (fp32, [B,T,H,64])
 *   kkt_scaled_dot      -> A (device only)
 *   kkt_solve_tril(A)   -> DIR/x_chain.bin  (fp32, [B,T,H,64])
 *   kkt_solve_gate_cumsum on DIR/g_raw.bin (per-token log-decays, in place)
 *                       -> DIR/x_gsum.bin, DIR/g_sum.bin
 * and exits 0, or prints the failing call and exits 1.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kkt_solve.h"

#define CHECK_HIP(call)                                                                    \
    do {                                                                                   \
        hipError_t e_ = (call);                                                            \
        if (e_ != hipSuccess) {                                                            \
            printf("%s failed: %s\n", #call, hipGetErrorString(e_));                       \
            return 1;                                                                      \
        }                                                                                  \
    } while (0)

#define CHECK_KKT(call)                                                                    \
    do {                                                                                   \
        kkt_status_t s_ = (call);                                                          \
        if (s_ != KKT_OK) {                                                                \
            printf("%s returned %d: %s\n", #call, (int)s_, kkt_last_error());              \
            return 1;                                                                      \
        }                                                                                  \
    } while (0)

static void* read_file(const char* dir, const char* name, size_t bytes)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "rb");
    if (f == NULL) return NULL;
    void* p = malloc(bytes);
    size_t got = (p != NULL) ? fread(p, 1, bytes, f) : 0;
    fclose(f);
    if (got != bytes) {
        free(p);
        return NULL;
    }
    return p;
}

static int write_file(const char* dir, const char* name, const void* p, size_t bytes)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "wb");
    if (f == NULL) return 1;
    size_t put = fwrite(p, 1, bytes, f);
    fclose(f);
    return put == bytes ? 0 : 1;
}

int main(int argc, char** argv)
{
    if (argc != 6) {
        printf("usage: %s DIR B T H K\n", argv[0]);
        return 1;
    }
    const char* dir = argv[1];
    const int64_t B = atoll(argv[2]), T = atoll(argv[3]), H = atoll(argv[4]), K = atoll(argv[5]);
    const size_t n_tok = (size_t)(B * T * H);
    const size_t k_bytes = n_tok * (size_t)K * 2, v_bytes = n_tok * 4, o_bytes = n_tok * 64 * 4;

    void* hk = read_file(dir, "k.bin", k_bytes);
    void* hg = read_file(dir, "g.bin", v_bytes);
    void* hb = read_file(dir, "beta.bin", v_bytes);
    void* hr = read_file(dir, "g_raw.bin", v_bytes);
    void* ho = malloc(o_bytes);
    void* hs = malloc(v_bytes);
    if (hk == NULL || hg == NULL || hb == NULL || hr == NULL || ho == NULL || hs == NULL) {
        printf("cannot read the inputs in %s\n", dir);
        return 1;
    }

    void *dk, *dg, *db, *dr, *dx, *dA;
    hipStream_t stream;
    CHECK_HIP(hipMalloc(&dk, k_bytes));
    CHECK_HIP(hipMalloc(&dg, v_bytes));
    CHECK_HIP(hipMalloc(&db, v_bytes));
    CHECK_HIP(hipMalloc(&dr, v_bytes));
    CHECK_HIP(hipMalloc(&dx, o_bytes));
    CHECK_HIP(hipMalloc(&dA, o_bytes));
    CHECK_HIP(hipStreamCreate(&stream));
    CHECK_HIP(hipMemcpy(dk, hk, k_bytes, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dg, hg, v_bytes, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(db, hb, v_bytes, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dr, hr, v_bytes, hipMemcpyHostToDevice));

    CHECK_KKT(kkt_solve(dk, (const float*)dg, (const float*)db, NULL, 0, B, T, H, K, 64,
                        KKT_DTYPE_BF16, KKT_DTYPE_F32, dx, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    CHECK_HIP(hipMemcpy(ho, dx, o_bytes, hipMemcpyDeviceToHost));
    if (write_file(dir, "x_fused.bin", ho, o_bytes)) return 1;

    CHECK_KKT(kkt_scaled_dot(dk, (const float*)dg, (const float*)db, NULL, 0, B, T, H, K, 64,
                             KKT_DTYPE_BF16, (float*)dA, stream));
    CHECK_KKT(kkt_solve_tril((const float*)dA, NULL, 0, B, T, H, 64, KKT_DTYPE_F32, dx, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    CHECK_HIP(hipMemcpy(ho, dx, o_bytes, hipMemcpyDeviceToHost));
    if (write_file(dir, "x_chain.bin", ho, o_bytes)) return 1;

    CHECK_KKT(kkt_solve_gate_cumsum(dk, (const float*)dr, (const float*)db, NULL, 0, B, T, H, K, 64,
                                    KKT_DTYPE_BF16, KKT_DTYPE_F32, dx, (float*)dr, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    CHECK_HIP(hipMemcpy(ho, dx, o_bytes, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(hs, dr, v_bytes, hipMemcpyDeviceToHost));
    if (write_file(dir, "x_gsum.bin", ho, o_bytes) || write_file(dir, "g_sum.bin", hs, v_bytes)) return 1;

    CHECK_HIP(hipStreamDestroy(stream));
    CHECK_HIP(hipFree(dk));
    CHECK_HIP(hipFree(dg));
    CHECK_HIP(hipFree(db));
    CHECK_HIP(hipFree(dr));
    CHECK_HIP(hipFree(dx));
    CHECK_HIP(hipFree(dA));
    free(hk);
    free(hg);
    free(hb);
    free(hr);
    free(ho);
    free(hs);
    printf("ok version %d\n", kkt_version());
    return 0;
}
