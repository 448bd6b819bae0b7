// Fused chunk-local KKT + triangular solve for MI355X (gfx950).
//
// Operation: MindSpeed-Ops pull request #135, "feat(triton): add
// chunk_gated_delta_rule_fwd_kkt_solve" (PR description; user-facing-change
// section; bot change summary).  For every 64-token chunk of every (batch
// row or sequence, head):
//   A[i][j] = beta_i (k_i . k_j) exp(clamp(g_i - g_j, -50, 50)) for i > j, 0 otherwise
//   out rows = rows of (I + A)^{-1}, 64 wide, written once in full.
//
// One wave64 owns one (chunk, head) tile from load to store; nothing goes
// back to HBM between the steps.
//   a1  tile -> (b, t0, L, h); for packed sequences a wave-wide prefix scan
//       over cu_seqlens (no host sync, no index tensor).
//   a2  K tile [64 x K] straight from HBM into VGPRs: lane (q, m) of the wave
//       holds row 16*bi + m of each 16-row block bi, 16 contiguous bytes per
//       MFMA k-step.  S = K K^T uses the same fragments as both operands, so
//       any fixed assignment of k indices to (lane group, slot) gives S.
//   a3  g and beta: one value per lane, shared through LDS.
//   a4  Gram on MFMA (bf16/f16: 16x16x32, fp32: 16x16x4), fp32 accumulate,
//       only the 10 lower 16x16 blocks.
//   a5  epilogue on the accumulators: beta row scale, clamped gate, strict
//       lower mask, all as selects so no inf*0 can appear.
//   a6  the four 16x16 unit-lower diagonal blocks inverted side by side by
//       forward substitution: lane (block, column) keeps one column in
//       VGPRs, row r needs rows < r only, all 15 steps unrolled (the pages'
//       static row loop and side-by-side 16x16 blocks, PyPTO GatedDeltaRule
//       case, sections 3.3.1, 3.3.2 and 3.4).
//   a7  the six off-diagonal 16x16 blocks, fp32 MFMA:
//         W_ik = X_ii A_ik                      (all six independent)
//         X_ij = -sum_{k=j}^{i-1} W_ik X_kj     (three dependency levels)
//       W is produced transposed (A_ik^T X_ii^T), which is the layout the
//       next product wants for its left operand; no shuffles are needed.
//   a8  each 16-row block row is staged through LDS and written as full
//       contiguous rows (256 B fp32 / 128 B bf16), upper zeros included.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <string>

#include "kkt_solve.h"

#define KKT_VERSION_NUMBER 100  // 0.1.0

namespace {

constexpr int kChunk = 64;
constexpr int kWave = 64;
constexpr int kWavesPerGroup = 4;
constexpr int kBlockLd = 20;   // padded row stride (floats) of a 16x16 LDS block
constexpr int kStageLd = 68;   // padded row stride (floats) of the 16x64 store stage
constexpr float kGateClamp = 50.0f;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Per-wave LDS.  The store stage reuses the diagonal-A area once the
// diagonal solve has read it.
struct WaveLds {
    float g[kChunk];
    float beta[kChunk];
    union {
        float adiag[4][16][kBlockLd];
        float stage[16][kStageLd];
    };
    float xdiag[4][16][kBlockLd];
};
static_assert(sizeof(float) * 4 * 16 * kBlockLd >= sizeof(float) * 16 * kStageLd, "stage fits");

// Orders this wave's LDS accesses: the compiler may not move memory
// operations across it, and the LDS executes one wave's operations in order.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------- element types
enum class Elt { F32, BF16, F16 };

template <Elt E> struct EltInfo;
template <> struct EltInfo<Elt::F32> { using storage = float; static constexpr int bytes = 4; };
template <> struct EltInfo<Elt::BF16> { using storage = uint16_t; static constexpr int bytes = 2; };
template <> struct EltInfo<Elt::F16> { using storage = uint16_t; static constexpr int bytes = 2; };

// fp32 -> bf16 bits, round to nearest even (the inputs are never NaN here).
__device__ __forceinline__ uint32_t bf16_bits_rne(float x)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t f16_bits_rne(float x)
{
    const _Float16 h = (_Float16)x;  // v_cvt_f16_f32 under the default round-to-nearest-even mode
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

template <Elt E> __device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <> __device__ __forceinline__ uint32_t pack2<Elt::BF16>(float lo, float hi)
{
    return bf16_bits_rne(lo) | (bf16_bits_rne(hi) << 16);
}
template <> __device__ __forceinline__ uint32_t pack2<Elt::F16>(float lo, float hi)
{
    return f16_bits_rne(lo) | (f16_bits_rne(hi) << 16);
}

// ---------------------------------------------------------------- MFMA helpers
// c += A B for 16x16x16 fp32 blocks.  a: lane (q, m) holds A[m][4q .. 4q+3];
// b: lane (q, n) holds B[4q .. 4q+3][n]; c: lane (q, n) holds C[4q .. 4q+3][n].
__device__ __forceinline__ f32x4 mm16(f32x4 a, f32x4 b, f32x4 c)
{
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
}

// One k-step of the Gram for a 16-byte fragment pair.
template <Elt E> __device__ __forceinline__ f32x4 gram_step(u32x4 a, u32x4 b, f32x4 c);
template <> __device__ __forceinline__ f32x4 gram_step<Elt::BF16>(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4 gram_step<Elt::F16>(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4 gram_step<Elt::F32>(u32x4 a, u32x4 b, f32x4 c)
{
    // reinterpret whole vectors: a bit-cast of a single vector element would
    // read the vector's first element instead
    const f32x4 af = __builtin_bit_cast(f32x4, a);
    const f32x4 bf = __builtin_bit_cast(f32x4, b);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(af[0], bf[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(af[1], bf[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(af[2], bf[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(af[3], bf[3], c, 0, 0, 0);
    return c;
}

// ---------------------------------------------------------------- tile map (a1)
struct Tile {
    int64_t row0;  // flat token index (b * T + t0) of the chunk's first row
    int len;       // valid rows L in [1, 64]; 0: no tile
    int h;
};

// Packed sequences: the chunk with global index c (chunks numbered sequence
// by sequence) is found with a wave-wide inclusive scan of per-sequence chunk
// counts, 64 sequences per pass.  Offsets are clamped into [0, T].
__device__ Tile varlen_tile(const int32_t* __restrict__ cu, int64_t num_seqs, int64_t T,
                            int64_t c, int h, int lane)
{
    Tile t{0, 0, h};
    int64_t before = 0;  // chunks in the sequences already passed
    for (int64_t base = 0; base < num_seqs; base += kWave) {
        const int64_t s = base + lane;
        int64_t bos = 0, eos = 0;
        if (s < num_seqs) {
            int64_t a = cu[s], e = cu[s + 1];
            bos = a < 0 ? 0 : (a > T ? T : a);
            eos = e < bos ? bos : (e > T ? T : e);
        }
        const int64_t n = (eos - bos + kChunk - 1) / kChunk;
        int64_t incl = n;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int64_t up = __shfl_up(incl, d, kWave);
            if (lane >= d) incl += up;
        }
        const bool hit = (s < num_seqs) && (before + incl > c);
        const uint64_t mask = __ballot(hit);
        if (mask != 0) {
            const int src = __builtin_ctzll(mask);
            const int64_t excl = incl - n;
            const int64_t sel_excl = __shfl(excl, src, kWave);
            const int64_t sel_bos = __shfl(bos, src, kWave);
            const int64_t sel_eos = __shfl(eos, src, kWave);
            const int64_t t0 = sel_bos + (c - before - sel_excl) * kChunk;
            const int64_t rem = sel_eos - t0;
            t.row0 = t0;
            t.len = (int)(rem < kChunk ? rem : kChunk);
            return t;
        }
        before += __shfl(incl, kWave - 1, kWave);
    }
    return t;
}

// ---------------------------------------------------------------- the kernel
template <Elt IN, Elt OUT, int K>
__global__ __launch_bounds__(kWave * kWavesPerGroup)
void kkt_solve_kernel(const typename EltInfo<IN>::storage* __restrict__ k,
                      const float* __restrict__ g, const float* __restrict__ beta,
                      const int32_t* __restrict__ cu_seqlens, int64_t num_seqs,
                      int64_t T, int H, int64_t chunks_per_row, int64_t n_tiles,
                      typename EltInfo<OUT>::storage* __restrict__ out)
{
    using in_t = typename EltInfo<IN>::storage;
    constexpr int kElemsPer16B = 16 / EltInfo<IN>::bytes;  // 8 (16-bit) or 4 (fp32)
    constexpr int kSteps = K / (4 * kElemsPer16B);          // 16-byte fragments per row per lane
    static_assert(K % (4 * kElemsPer16B) == 0, "K must fill whole fragments");

    __shared__ WaveLds lds_all[kWavesPerGroup];

    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int q = lane / 16;   // lane group (k-slot group of an MFMA operand)
    const int m = lane % 16;   // row inside a 16-row block (A operand) / column (D layout)
    WaveLds& lds = lds_all[wave];

    // XCD-aware order: workgroups are dispatched round-robin over the 8 XCDs;
    // give each XCD one contiguous range of tiles so that the heads of one
    // chunk (adjacent in memory) and their shared g/beta lines meet in one L2.
    const int64_t n_groups = gridDim.x;
    const int64_t hw = blockIdx.x;
    const int64_t xcd = hw % 8, slot = hw / 8;
    const int64_t per = n_groups / 8, extra = n_groups % 8;
    const int64_t group = (xcd < extra) ? xcd * (per + 1) + slot
                                        : extra * (per + 1) + (xcd - extra) * per + slot;
    const int64_t tile_id = group * kWavesPerGroup + wave;
    if (tile_id >= n_tiles) return;

    // ---- a1: tile map
    const int h = (int)(tile_id % H);
    const int64_t chunk = tile_id / H;
    Tile tile;
    if (cu_seqlens == nullptr) {
        const int64_t b = chunk / chunks_per_row;
        const int64_t c = chunk % chunks_per_row;
        const int64_t t0 = c * kChunk;
        tile.row0 = b * T + t0;
        tile.len = (int)((T - t0) < kChunk ? (T - t0) : kChunk);
        tile.h = h;
    } else {
        tile = varlen_tile(cu_seqlens, num_seqs, T, chunk, h, lane);
    }
    const int L = tile.len;
    if (L <= 0) return;  // wave-uniform

    // ---- a2: K fragments, all loads issued up front
    u32x4 frag[4][kSteps];
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
        const int r = 16 * bi + m;
        const in_t* src = k + ((tile.row0 + r) * H + h) * (int64_t)K + q * kElemsPer16B;
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (r < L) {
                v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + s * 4 * kElemsPer16B));
            }
            frag[bi][s] = v;
        }
    }

    // ---- a3: g and beta, one row per lane (rows >= L: gate 0, beta 0)
    {
        float gv = 0.0f, bv = 0.0f;
        if (lane < L) {
            const int64_t idx = (tile.row0 + lane) * H + h;
            gv = (g != nullptr) ? g[idx] : 0.0f;
            bv = (beta != nullptr) ? beta[idx] : 1.0f;
        }
        lds.g[lane] = gv;
        lds.beta[lane] = bv;
    }
    wave_lds_sync();
    const bool has_g = (g != nullptr);
    f32x4 g_row[4], b_row[4];
    float g_col[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        g_row[i] = *reinterpret_cast<const f32x4*>(&lds.g[16 * i + 4 * q]);
        b_row[i] = *reinterpret_cast<const f32x4*>(&lds.beta[16 * i + 4 * q]);
        g_col[i] = lds.g[16 * i + m];
    }

    // ---- a4 + a5: Gram blocks and epilogue.  Block (i, j): lane (q, n=m)
    // holds rows 16i + 4q + r, column 16j + n.
    auto epilogue = [&](f32x4 s, int i, int j) -> f32x4 {
        f32x4 a;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * i + 4 * q + r;
            const int col = 16 * j + m;
            float gate = 1.0f;
            if (has_g) {
                float d = g_row[i][r] - g_col[j];
                d = fminf(fmaxf(d, -kGateClamp), kGateClamp);
                gate = __expf(d);
            }
            const float v = b_row[i][r] * (s[r] * gate);
            a[r] = (row > col && row < L) ? v : 0.0f;
        }
        return a;
    };
    auto gram = [&](int i, int j) -> f32x4 {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < kSteps; ++s) acc = gram_step<IN>(frag[i][s], frag[j][s], acc);
        return acc;
    };

    // diagonal blocks go to LDS for the solve
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x4 a = epilogue(gram(i, i), i, i);
#pragma unroll
        for (int r = 0; r < 4; ++r) lds.adiag[i][4 * q + r][m] = a[r];
    }
    // off-diagonal blocks stay in VGPRs (layout: lane (q, n) = A_ij[4q + r][n])
    const f32x4 a10 = epilogue(gram(1, 0), 1, 0);
    const f32x4 a20 = epilogue(gram(2, 0), 2, 0);
    const f32x4 a21 = epilogue(gram(2, 1), 2, 1);
    const f32x4 a30 = epilogue(gram(3, 0), 3, 0);
    const f32x4 a31 = epilogue(gram(3, 1), 3, 1);
    const f32x4 a32 = epilogue(gram(3, 2), 3, 2);
    wave_lds_sync();

    // ---- a6: X_dd = (I + A_dd)^{-1}; lane (d = lane / 16, c = lane % 16)
    // computes column c of X_dd: x[r] = [r == c] - sum_{p < r} A[r][p] x[p].
    {
        const int d = lane / 16;
        const int c = lane % 16;
        float x[16];
        x[0] = (c == 0) ? 1.0f : 0.0f;
#pragma unroll
        for (int r = 1; r < 16; ++r) {
            float arow[16];
#pragma unroll
            for (int u = 0; u < (r + 3) / 4; ++u) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(&lds.adiag[d][r][4 * u]);
                arow[4 * u + 0] = v[0];
                arow[4 * u + 1] = v[1];
                arow[4 * u + 2] = v[2];
                arow[4 * u + 3] = v[3];
            }
            float acc = (r == c) ? 1.0f : 0.0f;
#pragma unroll
            for (int p = 0; p < r; ++p) acc = __builtin_fmaf(-arow[p], x[p], acc);
            x[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) lds.xdiag[d][r][c] = x[r];
    }
    wave_lds_sync();

    // X_dd in both operand layouts:
    //   xa[d]: lane (q, m) holds X_dd[m][4q .. 4q+3]   (left operand)
    //   xd[d]: lane (q, n) holds X_dd[4q .. 4q+3][n]   (right operand / result layout)
    f32x4 xa[4], xd[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        xa[d] = *reinterpret_cast<const f32x4*>(&lds.xdiag[d][m][4 * q]);
#pragma unroll
        for (int r = 0; r < 4; ++r) xd[d][r] = lds.xdiag[d][4 * q + r][m];
    }

    // ---- a8 helper: stage one 16-row block row and write full output rows
    using out_t = typename EltInfo<OUT>::storage;
    const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
    auto store_block_row = [&](int i, f32x4 b0, f32x4 b1, f32x4 b2, f32x4 b3) {
        wave_lds_sync();  // earlier stage reads (and the solve's adiag reads) are done
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            lds.stage[4 * q + r][0 + m] = b0[r];
            lds.stage[4 * q + r][16 + m] = b1[r];
            lds.stage[4 * q + r][32 + m] = b2[r];
            lds.stage[4 * q + r][48 + m] = b3[r];
        }
        wave_lds_sync();
        if constexpr (OUT == Elt::F32) {
            // 16 lanes per 256-byte row, 4 rows per pass
            const int rsub = lane / 16, c4 = (lane % 16) * 4;
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int rr = 4 * it + rsub;
                const int row = 16 * i + rr;
                const f32x4 v = *reinterpret_cast<const f32x4*>(&lds.stage[rr][c4]);
                if (row < L) {
                    float* dst = reinterpret_cast<float*>(out) + ((tile.row0 + row) * H + h) * (int64_t)kChunk + c4;
                    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst));
                }
            }
        } else {
            // 8 lanes per 128-byte row, 8 rows per pass
            const int rsub = lane / 8, c8 = (lane % 8) * 8;
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const int rr = 8 * it + rsub;
                const int row = 16 * i + rr;
                const f32x4 v0 = *reinterpret_cast<const f32x4*>(&lds.stage[rr][c8]);
                const f32x4 v1 = *reinterpret_cast<const f32x4*>(&lds.stage[rr][c8 + 4]);
                u32x4 p;
                p[0] = pack2<OUT>(v0[0], v0[1]);
                p[1] = pack2<OUT>(v0[2], v0[3]);
                p[2] = pack2<OUT>(v1[0], v1[1]);
                p[3] = pack2<OUT>(v1[2], v1[3]);
                if (row < L) {
                    out_t* dst = out + ((tile.row0 + row) * H + h) * (int64_t)kChunk + c8;
                    __builtin_nontemporal_store(p, reinterpret_cast<u32x4*>(dst));
                }
            }
        }
    };

    // block row 0 is final already
    store_block_row(0, xd[0], zero4, zero4, zero4);

    // ---- a7: merge.  wt_ik = (X_ii A_ik)^T; its result layout is the left
    // operand layout of W_ik.
    const f32x4 wt10 = mm16(a10, xa[1], zero4);
    const f32x4 wt20 = mm16(a20, xa[2], zero4);
    const f32x4 wt21 = mm16(a21, xa[2], zero4);
    const f32x4 wt30 = mm16(a30, xa[3], zero4);
    const f32x4 wt31 = mm16(a31, xa[3], zero4);
    const f32x4 wt32 = mm16(a32, xa[3], zero4);

    // X_ij = 0 - sum(...): exact negation that turns an all-zero sum into +0.0
    const f32x4 x10 = zero4 - mm16(wt10, xd[0], zero4);
    const f32x4 x21 = zero4 - mm16(wt21, xd[1], zero4);
    const f32x4 x32 = zero4 - mm16(wt32, xd[2], zero4);
    store_block_row(1, x10, xd[1], zero4, zero4);

    const f32x4 x20 = zero4 - mm16(wt21, x10, mm16(wt20, xd[0], zero4));
    const f32x4 x31 = zero4 - mm16(wt32, x21, mm16(wt31, xd[1], zero4));
    store_block_row(2, x20, x21, xd[2], zero4);

    const f32x4 x30 = zero4 - mm16(wt32, x20, mm16(wt31, x10, mm16(wt30, xd[0], zero4)));
    store_block_row(3, x30, x31, x32, xd[3]);
}

// ---------------------------------------------------------------- host side
thread_local std::string g_last_error;

kkt_status_t fail(kkt_status_t st, const std::string& msg)
{
    g_last_error = msg;
    return st;
}

// Per-device "is gfx950" cache: 0 unknown, 1 yes, 2 no.
constexpr int kMaxDevices = 64;
int g_arch_ok[kMaxDevices];
std::mutex g_arch_mutex;

kkt_status_t check_device(int* dev_out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(KKT_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(KKT_ERR_UNSUPPORTED, "device index out of range");
    std::lock_guard<std::mutex> lock(g_arch_mutex);
    if (g_arch_ok[dev] == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return fail(KKT_ERR_HIP, std::string("hipGetDeviceProperties: ") + hipGetErrorString(e));
        g_arch_ok[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    }
    if (g_arch_ok[dev] != 1) return fail(KKT_ERR_UNSUPPORTED, "device is not gfx950 (MI355X); this library is built for gfx950 only");
    *dev_out = dev;
    return KKT_OK;
}

kkt_status_t validate_cu_seqlens(const int32_t* cu, int64_t num_seqs, int64_t T, hipStream_t stream)
{
    std::string buf(sizeof(int32_t) * (size_t)(num_seqs + 1), '\0');
    int32_t* host = reinterpret_cast<int32_t*>(&buf[0]);
    hipError_t e = hipMemcpyAsync(host, cu, buf.size(), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fail(KKT_ERR_HIP, std::string("cu_seqlens copy: ") + hipGetErrorString(e));
    if (host[0] != 0) return fail(KKT_ERR_INVALID_ARGUMENT, "cu_seqlens[0] must be 0");
    for (int64_t s = 0; s < num_seqs; ++s) {
        if (host[s + 1] < host[s]) return fail(KKT_ERR_INVALID_ARGUMENT, "cu_seqlens must not decrease");
    }
    if (host[num_seqs] != T) return fail(KKT_ERR_INVALID_ARGUMENT, "cu_seqlens[num_seqs] must equal T");
    return KKT_OK;
}

template <Elt IN, Elt OUT, int K>
hipError_t launch(const void* k, const float* g, const float* beta, const int32_t* cu, int64_t num_seqs,
                  int64_t T, int64_t H, int64_t chunks_per_row, int64_t n_tiles, void* out,
                  hipStream_t stream)
{
    const int64_t groups = (n_tiles + kWavesPerGroup - 1) / kWavesPerGroup;
    hipLaunchKernelGGL((kkt_solve_kernel<IN, OUT, K>), dim3((unsigned)groups), dim3(kWave * kWavesPerGroup), 0,
                       stream, static_cast<const typename EltInfo<IN>::storage*>(k), g, beta, cu, num_seqs, T,
                       (int)H, chunks_per_row, n_tiles, static_cast<typename EltInfo<OUT>::storage*>(out));
    return hipGetLastError();
}

template <Elt IN, Elt OUT>
hipError_t launch_k(int64_t K, const void* k, const float* g, const float* beta, const int32_t* cu,
                    int64_t num_seqs, int64_t T, int64_t H, int64_t cpr, int64_t n_tiles, void* out,
                    hipStream_t stream)
{
    switch (K) {
    case 64: return launch<IN, OUT, 64>(k, g, beta, cu, num_seqs, T, H, cpr, n_tiles, out, stream);
    case 128: return launch<IN, OUT, 128>(k, g, beta, cu, num_seqs, T, H, cpr, n_tiles, out, stream);
    default: return launch<IN, OUT, 256>(k, g, beta, cu, num_seqs, T, H, cpr, n_tiles, out, stream);
    }
}

template <Elt IN>
hipError_t launch_out(kkt_dtype_t od, int64_t K, const void* k, const float* g, const float* beta,
                      const int32_t* cu, int64_t num_seqs, int64_t T, int64_t H, int64_t cpr, int64_t n_tiles,
                      void* out, hipStream_t stream)
{
    switch (od) {
    case KKT_DTYPE_F32: return launch_k<IN, Elt::F32>(K, k, g, beta, cu, num_seqs, T, H, cpr, n_tiles, out, stream);
    case KKT_DTYPE_BF16: return launch_k<IN, Elt::BF16>(K, k, g, beta, cu, num_seqs, T, H, cpr, n_tiles, out, stream);
    default: return launch_k<IN, Elt::F16>(K, k, g, beta, cu, num_seqs, T, H, cpr, n_tiles, out, stream);
    }
}

bool valid_dtype(int d) { return d == KKT_DTYPE_F32 || d == KKT_DTYPE_BF16 || d == KKT_DTYPE_F16; }

}  // namespace

extern "C" kkt_status_t kkt_solve(const void* k, const float* g, const float* beta,
                                  const int32_t* cu_seqlens, int64_t num_seqs,
                                  int64_t B, int64_t T, int64_t H, int64_t K,
                                  int64_t chunk_size, kkt_dtype_t in_dtype, kkt_dtype_t out_dtype,
                                  void* out, hipStream_t stream)
{
    g_last_error.clear();
    // ---- argument checks: no HIP call before they pass
    if (chunk_size != kChunk) return fail(KKT_ERR_UNSUPPORTED, "chunk_size must be 64");
    if (!valid_dtype((int)in_dtype) || !valid_dtype((int)out_dtype)) return fail(KKT_ERR_INVALID_ARGUMENT, "unknown dtype");
    if (B < 1 || H < 1 || K < 1 || T < 0) return fail(KKT_ERR_INVALID_ARGUMENT, "B, H, K must be >= 1 and T >= 0");
    if (K != 64 && K != 128 && K != 256) return fail(KKT_ERR_UNSUPPORTED, "K must be 64, 128 or 256");
    if (H > (int64_t)0x7FFFFFFF) return fail(KKT_ERR_INVALID_ARGUMENT, "H too large");
    if (cu_seqlens != nullptr && (B != 1 || num_seqs < 1)) {
        return fail(KKT_ERR_INVALID_ARGUMENT, "cu_seqlens needs B == 1 and num_seqs >= 1");
    }
    if (T == 0) return KKT_OK;
    if (k == nullptr || out == nullptr) return fail(KKT_ERR_INVALID_ARGUMENT, "k and out must not be NULL");

    const int64_t chunks_per_row = (T + kChunk - 1) / kChunk;
    // Packed sequences: at most floor(T/64) + num_seqs chunks; surplus waves exit.
    const int64_t n_chunks = (cu_seqlens == nullptr) ? B * chunks_per_row : T / kChunk + num_seqs;
    const int64_t n_tiles = n_chunks * H;
    const int64_t groups = (n_tiles + kWavesPerGroup - 1) / kWavesPerGroup;
    if (groups > 0x7FFFFFFFLL) return fail(KKT_ERR_INVALID_ARGUMENT, "problem too large for one launch");

    int dev = 0;
    kkt_status_t st = check_device(&dev);
    if (st != KKT_OK) return st;
    if (cu_seqlens != nullptr) {
        const char* v = getenv("KKT_VALIDATE");
        if (v != nullptr && v[0] == '1') {
            st = validate_cu_seqlens(cu_seqlens, num_seqs, T, stream);
            if (st != KKT_OK) return st;
        }
    }

    hipError_t e;
    switch (in_dtype) {
    case KKT_DTYPE_F32:
        e = launch_out<Elt::F32>(out_dtype, K, k, g, beta, cu_seqlens, num_seqs, T, H, chunks_per_row, n_tiles, out, stream);
        break;
    case KKT_DTYPE_BF16:
        e = launch_out<Elt::BF16>(out_dtype, K, k, g, beta, cu_seqlens, num_seqs, T, H, chunks_per_row, n_tiles, out, stream);
        break;
    default:
        e = launch_out<Elt::F16>(out_dtype, K, k, g, beta, cu_seqlens, num_seqs, T, H, chunks_per_row, n_tiles, out, stream);
        break;
    }
    if (e != hipSuccess) return fail(KKT_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
    return KKT_OK;
}

extern "C" const char* kkt_last_error(void) { return g_last_error.c_str(); }

extern "C" int kkt_version(void) { return KKT_VERSION_NUMBER; }
