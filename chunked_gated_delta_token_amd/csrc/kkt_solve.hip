// Fused chunk-local KKT + triangular solve for MI355X (gfx950).
//
// Operation: MindSpeed-Ops pull request #135, "feat(triton): add
// chunk_gated_delta_rule_fwd_kkt_solve" (PR description; user-facing-change
// section; bot change summary).  For every 64-token chunk of every (batch
// row or sequence, head):
//   A[i][j] = beta_i (k_i . k_j) exp(clamp(g_i - g_j, -50, 50)) for i > j, 0 otherwise
//   out rows = rows of (I + A)^{-1}, 64 wide, written once in full.
//
// One wave64 owns one (chunk, head) tile from load to store (on grids of at
// most 256 tiles two waves share it, kkt_solve_split_kernel); nothing goes
// back to HBM between the steps.
//   a1  tile -> (b, t0, L, h); for packed sequences a scan of (or, beyond
//       64 sequences, a 64-ary search over) cu_seqlens (no host sync, no
//       index tensor).  Every tensor of the
//       tile is then addressed through a buffer resource whose base is the
//       tile's first row and whose size ends after row L-1: loads of rows
//       >= L return 0 and stores to them are dropped by the hardware range
//       check, so no lane needs a bounds test or 64-bit address arithmetic.
//   a2  K tile [64 x K] straight from HBM into VGPRs: lane (q, m) of the wave
//       holds row 16*bi + m of each 16-row block bi, 16 contiguous bytes per
//       MFMA k-step.  S = K K^T uses the same fragments as both operands, so
//       any fixed assignment of k indices to (lane group, slot) gives S.
//   a3  g and beta: one row per lane.
//   a4  Gram on MFMA, 16x16x32 bf16/f16, fp32 accumulate, only the 10 lower
//       16x16 blocks.  fp32 keys are split into three bf16 parts (exact to
//       2^-27) and six part products are summed (split_bf16x3, gram_bf16x3):
//       fp32-level accuracy at 2.7 times fewer MFMA cycles than fp32 MFMA.
//   a5  epilogue on the accumulators.  When every gate value of the chunk
//       is within 25 of g_0, no pair differs by more than 50, the clamp
//       cannot bind, and exp(g_i - g_j) factors into exp(g_i - g_0)
//       exp(g_0 - g_j): each lane computes one row factor r = beta exp(g - g_0)
//       and one column factor c = exp(g_0 - g) for its own row, and every
//       element is (r_i S) c_j.  Otherwise every element takes the clamped exp
//       of its own difference.
//   a6  the four 16x16 unit-lower diagonal blocks inverted side by side by
//       forward substitution: lane (block, column) keeps one column in
//       VGPRs, all 15 steps unrolled (the pages' static row loop and
//       side-by-side 16x16 blocks, PyPTO GatedDeltaRule case, sections 3.3.1,
//       3.3.2 and 3.4).  The updates are right-looking (column p of A applied
//       to every later row as soon as x[p] is final), so the dependent chain is
//       one FMA per row; A[r][p] reaches the lanes of a block by a DPP row
//       broadcast inside the FMA.
//   a7  the six off-diagonal 16x16 blocks, fp32 MFMA:
//         W_ik = X_ii A_ik                      (all six independent)
//         X_ij = -sum_{k=j}^{i-1} W_ik X_kj     (three dependency levels)
//       W is produced transposed (A_ik^T X_ii^T), which is the layout the
//       next product wants for its left operand; no shuffles are needed.
//   a8  each 16-row block row is staged through LDS and written as full
//       contiguous rows (256 B fp32 / 128 B bf16), upper zeros included.
//
// The same per-wave pipeline (chunk_rows) also serves the unfused chain's two
// steps (ScaledDot: a1-a5 and A written in fp32; SolveTril: A read back, then
// a6-a8), the gate formed from per-token log-decays (a wave scan before a4),
// and 128-token chunks (kkt_solve128_kernel: the two 64-row halves plus the
// block below the diagonal, one workgroup per chunk), and, split between two
// waves of a workgroup, the small grids of the fused op, its gate-sum form and
// the solve of a given A (the same operations in the same order, so the same
// bits).
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <string>

#include "kkt_solve.h"

#define KKT_VERSION_NUMBER 904  // 0.9.4

namespace {

constexpr int kChunk = 64;
constexpr int kWave = 64;
constexpr int kWavesPerGroup = 4;
constexpr int kBlockLd = 20;   // padded row stride (floats) of a 16x16 LDS block
constexpr int kStageLd = 68;   // padded row stride (floats) of the 16x64 store stage
constexpr float kGateClamp = 50.0f;
// buffer resource word 3 for raw (untyped) buffer access on gfx9-family GPUs
constexpr int kRawBufferFlags = 0x00020000;
constexpr int kNonTemporal = 2;  // cache-policy bit "nt" of a buffer access

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Per-wave LDS.  The gate epilogue's per-row values; then one 16x16x4 area
// that holds, in turn, the diagonal blocks of A, the diagonal inverses, and
// the store stage of each block row.
struct GateLds {
    float row_scale[kChunk];  // r (factored gate) or beta (clamped gate)
    float col_scale[kChunk];  // c (factored gate), or a column gate
    float gate[kChunk];       // g (clamped gate)
};
struct WaveLds : GateLds {
    union {
        float blk[4][16][kBlockLd];
        float stage[16][kStageLd];
    };
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

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRawBufferFlags);
}

// Key pieces of a kernel built for K_T.  A call takes the smallest K_T >= K,
// and the key bytes beyond the row's K * element size must enter the Gram as
// zeros.  A kernel built for K_T serves the K in (K_T / 2, K_T] (K_T = 64:
// every K up to 64) whose rows are whole 16-byte pieces.
//   - k-step s (64 bytes of a row: a 16-byte piece per lane group q) is read
//     through the tile's resource when it starts inside the row, and through
//     one of zero length (every load returns 0) when it starts at or beyond
//     the row's end: a scalar select per step (K is uniform).  The steps
//     below the smallest K this kernel serves with whole steps, K_T / 2 plus
//     one step, take no select.
//   - A row that ends inside a k-step (`ragged`: 16-bit K not a multiple of
//     32, fp32 K not a multiple of 16) reads that step whole, into the next
//     key row or past the resource's end (zeros); once the loads have
//     arrived, the lane groups whose piece lies past the row's end are
//     zeroed (mask_key_tail, a uniform branch taken only for such K).
// (Selecting per-lane offsets before the loads instead cost 0.3-0.4 us of
// 7.7 on (1,8192,8,128), with or without a branch around them: the compiler
// then scheduled the tile's loads worse, or waited for g and beta first.)
template <int K_T, int ELT_BYTES>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t k_step_rsrc(__amdgpu_buffer_rsrc_t r, int s, uint32_t k_head_bytes)
{
    constexpr int kAlways = (K_T == 64) ? 1 : K_T * ELT_BYTES / 128 + 1;
    if (s < kAlways) return r;
    return ((uint32_t)s * 64u < k_head_bytes) ? r : __builtin_amdgcn_make_buffer_rsrc(nullptr, 0, 0, kRawBufferFlags);
}

// Key fragments f[b][s]: 16 bytes of the row at byte offset voff[b] (the
// lane's piece in k-step 0) at k-step s0 + s, issued block by block.
template <int K_T, int ELT_BYTES, int NB, int NS>
__device__ __forceinline__ void load_key_frags(u32x4 (&f)[NB][NS], __amdgpu_buffer_rsrc_t r, const uint32_t (&voff)[NB],
                                               int s0, uint32_t k_head_bytes)
{
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            f[b][s] = __builtin_amdgcn_raw_buffer_load_b128(k_step_rsrc<K_T, ELT_BYTES>(r, s0 + s, k_head_bytes),
                                                            voff[b] + (s0 + s) * 64, 0, 0);
        }
    }
}

// Zero the pieces of f (k-steps s0 ..) that lie past the row's end, when the
// row ends inside a k-step.  Waits for the fragments.
template <int K_T, int ELT_BYTES, int NB, int NS>
__device__ __forceinline__ void mask_key_tail(u32x4 (&f)[NB][NS], int s0, int q, uint32_t k_head_bytes)
{
    if ((k_head_bytes & 63u) == 0) return;
    constexpr int kFirst = (K_T == 64) ? 0 : (K_T / 2) * ELT_BYTES / 64;  // earliest step a row can end in
    const int sp = (int)(k_head_bytes >> 6);                              // the step it ends in
    const bool keep = (uint32_t)(q * 16) < (k_head_bytes & 63u);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        if (s0 + s < kFirst || s0 + s != sp) continue;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (!keep) f[b][s] = u32x4{0u, 0u, 0u, 0u};
        }
    }
}

// ---------------------------------------------------------------- element types
enum class Elt { F32, BF16, F16 };

// What one launch computes.
//   Fused:     k, g, beta -> (I + A)^{-1}            (the fused op)
//   ScaledDot: k, g, beta -> A, fp32                 (first step of the unfused chain)
//   SolveTril: A (fp32)   -> (I + strict_lower(A))^{-1}  (second step)
enum class Mode { Fused, ScaledDot, SolveTril };

template <Elt E> struct EltInfo;
template <> struct EltInfo<Elt::F32> { using storage = float; static constexpr int bytes = 4; };
template <> struct EltInfo<Elt::BF16> { using storage = uint16_t; static constexpr int bytes = 2; };
template <> struct EltInfo<Elt::F16> { using storage = uint16_t; static constexpr int bytes = 2; };

// Two fp32 values -> packed 16-bit pair (low half first), rounded to nearest
// even by the hardware converts (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32 under
// the default round-to-nearest-even mode).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <Elt E> __device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <> __device__ __forceinline__ uint32_t pack2<Elt::BF16>(float lo, float hi)
{
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
template <> __device__ __forceinline__ uint32_t pack2<Elt::F16>(float lo, float hi)
{
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
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

// One k-step of the Gram for a 16-byte fragment pair of 16-bit keys (fp32
// keys go through split_bf16x3 / gram_bf16x3 below).
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


// fp32 keys on the 16-bit matrix cores.  Eight fp32 values (two fragments)
// become three bf16 parts, x = hi + mid + lo + e with |e| <= 2^-27 |x|: each
// part is the round-to-nearest-even bf16 of what the parts before it leave,
// and each remainder is exact in fp32.  (Eight values per lane make one k-slot
// set of a 16x16x32 MFMA; the two Gram operands use the same set, so their
// product sums the same k.)
struct Bf16x3 {
    bf16x8 hi, mid, lo;
};

__device__ __forceinline__ Bf16x3 split_bf16x3(u32x4 a0, u32x4 a1)
{
    const f32x4 x0 = __builtin_bit_cast(f32x4, a0);
    const f32x4 x1 = __builtin_bit_cast(f32x4, a1);
    float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    u32x4 part[3];
#pragma unroll
    for (int p = 0; p < 3; ++p) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // one hardware convert packs two values; their fp32 values are
            // the packed halves moved to the top of a word
            const uint32_t w = pack2<Elt::BF16>(x[2 * e], x[2 * e + 1]);
            part[p][e] = w;
            if (p < 2) {
                x[2 * e] -= __builtin_bit_cast(float, w << 16);
                x[2 * e + 1] -= __builtin_bit_cast(float, w & 0xffff0000u);
            }
        }
    }
    return Bf16x3{__builtin_bit_cast(bf16x8, part[0]), __builtin_bit_cast(bf16x8, part[1]),
                  __builtin_bit_cast(bf16x8, part[2])};
}

// c += A B^T over one 32-wide k-slot set of split fp32 rows: the six part
// products down to order 2^-18 |a||b| (the three left out are below
// 2^-26 |a||b|), smallest first.
__device__ __forceinline__ f32x4 gram_bf16x3(const Bf16x3& a, const Bf16x3& b, f32x4 c)
{
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.mid, b.mid, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.mid, b.hi, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.mid, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, c, 0, 0, 0);
    return c;
}

// ---------------------------------------------------------------- launch arguments
// How workgroups map to tiles.  The hardware hands workgroups to the 8 XCDs
// round-robin (workgroup w runs on XCD w % 8), and each XCD has its own L2.
//   kHardwareOrder:   tile group = workgroup index.
//   kContiguous:      each XCD takes one contiguous range of tile groups.
//   kChunkRoundRobin: runs of 2^log2_group_run consecutive workgroups (the
//                     ones that cover the heads of one chunk, when that count
//                     is a power of two) run on one XCD, one after another,
//                     and the runs go round-robin over the XCDs.  The heads of
//                     a token share cache lines of g, beta (and the summed
//                     gate), so each such line is then fetched and written by
//                     one L2.
enum XcdOrder { kHardwareOrder = 0, kContiguous = 1, kChunkRoundRobin = 2 };

// Unsigned division by a launch constant d >= 1 for dividends n < 2^31, as a
// multiply-high and a shift (set up on the host by make_fastdiv):
//   d a power of two:  magic = 0, n / d = n >> shift;
//   otherwise:         shift = floor(log2 d), magic = ceil(2^(32 + shift) / d)
//                      (in (2^31, 2^32) since 2^shift < d < 2^(shift+1)),
//                      n / d = mulhi(n, magic) >> shift.
// Exact: with magic = (2^(32+s) + e) / d, 0 <= e < d < 2^(s+1), the estimate
// exceeds n / d by n e / (d 2^(32+s)) < 2^31 2^(s+1) / (d 2^(32+s)) = 1 / d,
// which never carries past the next integer since frac(n / d) <= 1 - 1 / d.
struct FastDiv {
    uint32_t magic;
    uint32_t shift;
};

__device__ __forceinline__ uint32_t fast_div(uint32_t n, FastDiv d)
{
    return (d.magic == 0) ? (n >> d.shift) : (__umulhi(n, d.magic) >> d.shift);
}

struct KernelArgs {
    const void* k;
    const float* g;
    const float* beta;
    const int32_t* cu_seqlens;  // nullptr: fixed-length rows
    void* out;
    int64_t T;                  // tokens per batch row (total packed tokens for varlen)
    int32_t num_seqs;
    int32_t H;
    int32_t n_tiles;            // tiles in the grid (an upper bound for varlen)
    uint32_t n_groups;          // workgroups in the grid
    uint32_t k_row_bytes;       // bytes between consecutive tokens of one head in k
    uint32_t o_row_bytes;       // bytes between consecutive tokens of one head in out
    int32_t xcd_order;          // workgroup -> tile order, one of the XcdOrder values
    int32_t log2_group_run;     // kChunkRoundRobin: log2 of the workgroups kept together on one XCD
    uint32_t remap_groups;      // kChunkRoundRobin: workgroups in whole rounds (the rest keep their order)
    float* g_out;               // gate-sum kernel: where the summed gate goes, or nullptr
    int32_t split_tiles;        // host only: launch the fused op's two-wave-per-tile form
    int32_t tile_waves;         // one-wave-per-tile kernels: waves (tiles) per workgroup, 1 or 4
    uint32_t k_head_bytes;      // bytes of one key row of one head (K * element size, a multiple of
                                // 16); the kernel's template K may be larger: further pieces read as 0
    FastDiv div_H;              // division by H (tile -> chunk, head)
    FastDiv div_chunks;         // division by chunks_per_row (chunk -> batch row, chunk in row)
    int32_t gate_gather;        // gate-sum kernel: the four tiles of a workgroup (four heads of one
                                // chunk) write their summed gates together (run_tile)
    int32_t packed;             // cu_seqlens != nullptr, preloaded: the tile map tests this flag,
                                // not the pointer, so fixed-length rows never wait for the pointer
};

// Kernel arguments, preloaded.  Every tile needs the fields below before it
// can issue its first load (workgroup order, tile map, the key, g, beta and
// output addresses) or during its compute (the gate-sum output).  Passed as
// the leading 9 scalar kernel arguments (14 dwords), they are preloaded into
// SGPRs when the wave launches (the library is built with
// -amdgpu-kernarg-preload-count=9); read from the kernel argument segment,
// they would cost a tile one scalar-load round trip, about 0.5 us at the
// start of a launch, before its loads or in the middle of its compute (the
// next LDS wait waits for it too).  The other fields (packed sequences,
// options) come from the KernelArgs copy behind them.
// The five addresses are below 2^48 (setup() checks it; buffer resources
// hold 48-bit bases); their top 16 bits carry the small fields:
//   k:    xcd_order (bits 0-1), log2_group_run (2-6), tile_waves (7-9,
//         1 or 4), div_H.shift (10-14), packed (15);
//   g:    div_chunks.magic, low half;  beta: its high half;
//   out:  div_chunks.shift (0-4), log2 of the output bytes of one head's
//         row minus 7 (5-6), k_head_bytes / 16 (7-13), gate_gather (14).
// n_groups, remap_groups, k_row_bytes and o_row_bytes follow from the
// others (launch() checks the n_groups they give).
#define KKT_KERNEL_PARAMS                                                                                      \
    uint64_t pre_k, uint64_t pre_g, uint64_t pre_beta, uint64_t pre_out, uint64_t pre_g_out, uint32_t pre_n_tiles, \
        uint32_t pre_H, uint32_t pre_div_H, uint32_t pre_T, const KernelArgs args_in
#define KKT_KERNEL_ARGS                                                                                        \
    const KernelArgs args = with_preloaded(args_in, pre_k, pre_g, pre_beta, pre_out, pre_g_out, pre_n_tiles,  \
                                           pre_H, pre_div_H, pre_T)

constexpr uint64_t kAddrMask = (1ull << 48) - 1;

__device__ __forceinline__ KernelArgs with_preloaded(KernelArgs a, uint64_t k, uint64_t g, uint64_t beta,
                                                     uint64_t out, uint64_t g_out, uint32_t n_tiles, uint32_t H,
                                                     uint32_t div_H, uint32_t T)
{
    const uint32_t fk = (uint32_t)(k >> 48), fg = (uint32_t)(g >> 48), fb = (uint32_t)(beta >> 48),
                   fo = (uint32_t)(out >> 48);
    a.k = reinterpret_cast<const void*>(k & kAddrMask);
    a.g = reinterpret_cast<const float*>(g & kAddrMask);
    a.beta = reinterpret_cast<const float*>(beta & kAddrMask);
    a.out = reinterpret_cast<void*>(out & kAddrMask);
    a.g_out = reinterpret_cast<float*>(g_out & kAddrMask);
    a.xcd_order = (int32_t)(fk & 3u);
    a.log2_group_run = (int32_t)((fk >> 2) & 31u);
    a.tile_waves = (int32_t)((fk >> 7) & 7u);
    a.div_H = FastDiv{div_H, (fk >> 10) & 31u};
    a.packed = (int32_t)((fk >> 15) & 1u);
    a.div_chunks = FastDiv{fg | (fb << 16), fo & 31u};
    a.o_row_bytes = H << (7u + ((fo >> 5) & 3u));
    a.k_head_bytes = ((fo >> 7) & 127u) * 16u;
    a.gate_gather = (int32_t)((fo >> 14) & 1u);
    a.n_tiles = (int32_t)n_tiles;
    a.H = (int32_t)H;
    a.T = (int64_t)T;
    a.k_row_bytes = H * a.k_head_bytes;
    // tile_waves is 1 or 4 (the shift by tile_waves / 2 divides by it)
    const uint32_t tw = (uint32_t)a.tile_waves;
    a.n_groups = (n_tiles + tw - 1u) >> (tw >> 1);
    const uint32_t lg = (uint32_t)a.log2_group_run;
    a.remap_groups = (a.n_groups >> (lg + 3u)) << (lg + 3u);
    return a;
}

// ---------------------------------------------------------------- tile map (a1)
struct Tile {
    int64_t row0;  // flat token index (b * T + t0) of the chunk's first row
    int len;       // valid rows L in [1, 64]; 0: no tile
};

// Packed sequences: grid slot w -> (first row, valid rows).  The grid has
// T / CH + num_seqs slots, an upper bound on the chunk count.
//   Up to 64 sequences: slots are the chunks numbered sequence by sequence;
//   one wave-wide inclusive scan of the per-sequence chunk counts finds the
//   sequence.  Slots beyond the last chunk are empty.
//   More sequences: slots are numbered so that a slot can be found from the
//   offsets alone: sequence s owns [S(s), S(s) + ceil(len_s / CH)) with
//   S(s) = floor(bos_s / CH) + s.  S is strictly increasing, the ranges do
//   not overlap and end below T / CH + num_seqs; slots in no range are empty.
//   Slot w belongs to the last sequence with S(s) <= w, found by a 64-ary
//   search (each level probes 64 evenly spaced sequences, one per lane), so
//   the search takes ceil(log64(num_seqs)) dependent rounds of loads instead
//   of a scan over every sequence before the chunk.
// Offsets are clamped into [0, T] (they are int32, so every clamped offset
// fits in 32 bits).
template <int CH>
__device__ Tile varlen_tile(const int32_t* __restrict__ cu, int32_t num_seqs, int64_t T, int32_t w, int lane)
{
    const int32_t t_max = T < INT32_MAX ? (int32_t)T : INT32_MAX;
    Tile t{0, 0};
    auto clamped = [&](int32_t s, int32_t& bos, int32_t& eos) {
        const int32_t a = cu[s], e = cu[s + 1];
        bos = a < 0 ? 0 : (a > t_max ? t_max : a);
        eos = e < bos ? bos : (e > t_max ? t_max : e);
    };
    if (num_seqs <= kWave) {
        int32_t bos = 0, eos = 0;
        if (lane < num_seqs) clamped(lane, bos, eos);
        const int32_t n = (eos - bos + CH - 1) / CH;
        int32_t incl = n;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int32_t up = __shfl_up(incl, d, kWave);
            if (lane >= d) incl += up;
        }
        const uint64_t mask = __ballot(lane < num_seqs && incl > w);
        if (mask == 0) return t;
        const int src = __builtin_ctzll(mask);
        const int32_t sel_excl = __shfl(incl - n, src, kWave);
        const int32_t sel_bos = __shfl(bos, src, kWave);
        const int32_t sel_eos = __shfl(eos, src, kWave);
        const int64_t t0 = sel_bos + (int64_t)(w - sel_excl) * CH;
        const int64_t rem = sel_eos - t0;
        t.row0 = t0;
        t.len = (int)(rem < CH ? rem : CH);
        return t;
    }
    int32_t lo = 0, span = num_seqs;  // the sequence sought lies in [lo, lo + span)
    for (;;) {
        const int32_t step = (span + kWave - 1) / kWave;
        const int32_t s = lo + lane * step;
        int32_t bos = 0, eos = 0;
        bool le = false;
        if (lane * step < span) {
            clamped(s, bos, eos);
            le = (int64_t)(bos / CH) + s <= w;
        }
        const uint64_t mask = __ballot(le);
        if (mask == 0) return t;  // (only with offsets that do not start at 0)
        const int src = 63 - __builtin_clzll(mask);
        const int32_t end = lo + span;
        lo += src * step;
        span = (end - lo < step) ? end - lo : step;
        if (span <= 1) {
            const int32_t sel_bos = __shfl(bos, src, kWave);
            const int32_t sel_eos = __shfl(eos, src, kWave);
            const int64_t t0 = sel_bos + (int64_t)(w - sel_bos / CH - lo) * CH;
            if (t0 < sel_eos) {
                const int64_t rem = sel_eos - t0;
                t.row0 = t0;
                t.len = (int)(rem < CH ? rem : CH);
            }
            return t;
        }
    }
}

// Workgroup order (see XcdOrder); both remaps are permutations of
// [0, n_groups).  Computed without branches from preloaded kernel arguments
// only (KKT_KERNEL_PARAMS), so no memory round trip comes before the tile's
// first loads.
__device__ __forceinline__ uint32_t workgroup_order(const KernelArgs& args)
{
    const uint32_t n_groups = args.n_groups;
    const uint32_t hw = blockIdx.x;
    const uint32_t xcd = hw % 8, slot = hw / 8;
    const uint32_t per = n_groups / 8, extra = n_groups % 8;
    const uint32_t g_contiguous =
        (xcd < extra) ? xcd * (per + 1) + slot : extra * (per + 1) + (xcd - extra) * per + slot;
    const int lg = args.log2_group_run;
    const uint32_t g_runs = (hw < args.remap_groups)
        ? ((((slot >> lg) << 3) + xcd) << lg) | (slot & ((1u << lg) - 1u)) : hw;
    return (args.xcd_order == kContiguous) ? g_contiguous
         : (args.xcd_order == kChunkRoundRobin) ? g_runs : hw;
}

// Chunk c of CH tokens of one head -> (first row, valid rows); the result is
// wave-uniform and lives in scalar registers.
template <int CH>
__device__ __forceinline__ Tile chunk_tile(const KernelArgs& args, uint32_t chunk, int lane)
{
    Tile tile;
    if (!args.packed) {
        const uint32_t chunks_per_row = (uint32_t)((args.T + (CH - 1)) / CH);
        const uint32_t b = fast_div(chunk, args.div_chunks);
        const uint32_t c = chunk - b * chunks_per_row;
        const int64_t t0 = (int64_t)c * CH;
        tile.row0 = (int64_t)b * args.T + t0;
        tile.len = (int)((args.T - t0) < CH ? (args.T - t0) : CH);
    } else {
        tile = varlen_tile<CH>(args.cu_seqlens, args.num_seqs, args.T, (int32_t)chunk, lane);
    }
    tile.len = __builtin_amdgcn_readfirstlane(tile.len);
    tile.row0 = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(tile.row0 >> 32)) << 32) |
                          (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)tile.row0));
    return tile;
}

// LDS of one 128-token tile (one workgroup), in two overlapping layouts.
// Until the workgroup barrier that ends the first phase: the waves' own
// areas and the first half's key fragments as wave 0 loaded them (for waves
// 2 and 3).  After it: the blocks the waves exchange (X11, X22, A21, then P
// and X21).  39,424 bytes: four workgroups fit in a CU's 160 KB.
struct Chunk128Lds {
    union {
        struct {
            WaveLds half[2];                   // waves 0 and 1 (the 64-row pipelines)
            GateLds cross_gate[2];             // waves 2 and 3 (the A21 epilogue)
            u32x4 kimg[4][4][kWave];           // rows 0..63: key fragments (16-row block, k-step, lane)
        };
        struct {
            float x22[10][16][kBlockLd];       // X22 blocks, row-major: x22[b][row][col]
            union {
                struct {
                    f32x4 x11[10][kWave];      // X11 blocks, result-layout register images
                    f32x4 a21[16][kWave];      // A21 blocks (left-operand layout), then P blocks (result layout)
                } cross;
                float x21[kChunk][kStageLd];   // X21 rows staged for the store
            };
        };
    };
};
static_assert(sizeof(Chunk128Lds) * 4 <= 160 * 1024, "four 128-token workgroups per CU");

// Index of lower block (i, j), j <= i, of a 4x4 block-triangular matrix.
__host__ __device__ constexpr int tri(int i, int j) { return i * (i + 1) / 2 + j; }

// Inclusive prefix sum over the 64 lanes of a wave, in fp32 (a 6-level tree).
// Every wave that needs a chunk's summed gate uses this one function, so the
// same decays give the same bits wherever they are summed.
__device__ __forceinline__ float wave_prefix_sum(float v, int lane)
{
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const float up = __shfl_up(v, d, kWave);
        if (lane >= d) v += up;
    }
    return v;
}

// ---------------------------------------------------------------- the kernel
// Steps a2-a8 for 64 rows of one chunk of CH tokens, on one wave.  CH = 64:
// the whole chunk (half = 0).  CH = 128: rows 64*half .. 64*half+63, the
// half's own diagonal 64x64 block of the inverse; its columns go to
// 64*half .. 64*half+63 of the 128-wide output rows (half 0 also writes the
// zeros of columns 64..127), and the block is left in ex for the rest of the
// workgroup.  tok: flat (token, head) index of the chunk's first row; L: valid
// rows of the chunk.
// GATE_SUM: g holds per-token log-decays that the tile sums itself (a
// separate instantiation, so the plain fused kernel carries none of it).
// CH = 128: before it leaves X11 / X22 in ex the wave waits at the workgroup
// barrier that ends the first phase (the exchange area overlaps the
// first-phase areas).  SHARE: after its Gram, wave 0 also writes its key
// fragments to ex->kimg for the A21 waves, and both waves take part in the
// barrier that makes them visible.
// SPLIT: 0, the wave does the whole 64-token tile; 1 or 2, the first or
// second wave of a tile split over two waves (kkt_solve_split_kernel).  The
// first wave forms the diagonal blocks and block rows 1 and 2 of A, inverts
// all four diagonal blocks and finishes block rows 0..2; the second forms
// A30, A31, A32 meanwhile and finishes block row 3.  They exchange the
// diagonal inverses and X10, X21, X20 through LDS at three workgroup
// barriers.  Every block is formed by the same operations in the same order
// as in the one-wave tile, so the results are bit-identical.
// blk: the diagonal-block area (lds.blk for one wave; shared by the two waves
// of a split tile); xchg: the split tile's exchange area (else unused).
template <Mode MODE, Elt IN, Elt OUT, int K, bool GATE_SUM, int CH, bool SHARE = false, int SPLIT = 0>
__device__ __forceinline__ void chunk_rows(const KernelArgs& args, WaveLds& lds, float (&blk)[4][16][kBlockLd],
                                           f32x4 (*xchg)[kWave], int lane, int64_t tok, int L,
                                           int half, Chunk128Lds* ex)
{
    constexpr int kInBytes = EltInfo<IN>::bytes;
    constexpr int kOutBytes = EltInfo<OUT>::bytes;
    constexpr int kElemsPer16B = 16 / kInBytes;            // 8 (16-bit) or 4 (fp32)
    constexpr int kSteps = K / (4 * kElemsPer16B);          // 16-byte fragments per row per lane
    static_assert(K % (4 * kElemsPer16B) == 0, "K must fill whole fragments");
    static_assert(CH == 64 || (CH == 128 && MODE == Mode::Fused), "128-token chunks: fused op only");
    static_assert(!SHARE || (CH == 128 && kSteps <= 4), "shared key tile: 128-token kernel, at most 4 k-steps");
    static_assert(SPLIT == 0 || (CH == 64 && MODE != Mode::ScaledDot), "split tiles: the 64-token solve");
    // diagonal blocks this wave inverts (the first wave of a split tile
    // inverts all four, while the second forms its row's other blocks)
    auto owns = [](int) { return SPLIT != 2; };
    const int q = lane / 16;   // lane group (k-slot group of an MFMA operand)
    const int m = lane % 16;   // row inside a 16-row block (A operand) / column (D layout)
    const int H = args.H;
    // first row and first output column of this wave's 64 rows
    const uint32_t row_base = (CH == 128) ? 64u * (uint32_t)half : 0u;
    const uint32_t col_base = row_base;

    // split tile, GATE_SUM: the summed gate of row `lane`, written to g_out by
    // the first wave once the second has read the decays (g_out may be g)
    float g_sum = 0.0f;
    (void)g_sum;

    bool diag_in_lds = false;  // the diagonal blocks already written to blk
    // The 10 lower 16x16 blocks of A, result layout: A[i][j] lane (q, n)
    // holds A_ij[4q .. 4q+3][n] (rows 16i + 4q + r, column 16j + n).  The
    // diagonal blocks still hold their upper part here; it is masked below.
    f32x4 A[4][4];
    if constexpr (MODE == Mode::SolveTril) {
        // ---- A from memory (fp32 rows of 64; the kernel argument k carries A)
        // The first row of a diagonal block has no strictly lower entry in
        // it: those lanes read past the resource's end (zeros, no memory
        // access), so rows 0 and 32, whose lines no other block of their
        // row touches, cost no fetch.  (The range is below 2^31: the host
        // checks chunk * row stride.)
        const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(
            static_cast<const char*>(args.k) + tok * (int64_t)(CH * 4),
            (uint32_t)(L - 1) * args.k_row_bytes + CH * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int j = 0; j <= i; ++j) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    uint32_t voff = (uint32_t)(16 * i + 4 * q + r) * args.k_row_bytes + (16 * j + m) * 4;
                    if (j == i && r == 0 && q == 0) voff = 0x80000000u;
                    const float a = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(a_rsrc, voff, 0, 0));
                    A[i][j][r] = a;
                }
            }
        }
    } else {
        const bool has_g = args.g != nullptr;
        const bool valid = lane < L - (int)row_base;
        float gv = 0.0f, bv = 1.0f, g_first = 0.0f;
        u32x4 frag[4][kSteps];
        const __amdgpu_buffer_rsrc_t k_rsrc = make_rsrc(
            static_cast<const char*>(args.k) + tok * (int64_t)args.k_head_bytes,
            (uint32_t)(L - 1) * args.k_row_bytes + args.k_head_bytes);

        // Byte offsets of this lane's key pieces in k-step 0 of each 16-row
        // block.  One tile per wave: fixed here, before any load is in
        // flight (formed later, one 32-bit multiply-add became a 64-bit one
        // whose unused upper addend was allotted a register a g or beta load
        // was still filling, and the wave then waited for that load before
        // issuing its key loads; (1,8192,8,128) 7.8 -> 7.5 us).  Two-wave
        // tiles form them at the loads: hoisted, their small grids took
        // 0.58 us longer (4.38 -> 4.96 us on 32 tiles).
        uint32_t key_voff[4];
        auto key_offsets = [&] {
#pragma unroll
            for (int bi = 0; bi < 4; ++bi) key_voff[bi] = (row_base + (uint32_t)(16 * bi + m)) * args.k_row_bytes + q * 16;
        };
        if constexpr (SPLIT == 0) {
            key_offsets();
#pragma unroll
            for (int bi = 0; bi < 4; ++bi) asm volatile("" : "+v"(key_voff[bi]));
        }

        // ---- a3: g and beta, one row per lane (rows >= L read as 0).  Issued
        // before the K tile: loads complete in order, so waiting for these two
        // does not wait for the whole tile.
        {
            const uint32_t voff = (row_base + (uint32_t)lane) * (uint32_t)H * 4u;
            const uint32_t span = (uint32_t)(L - 1) * (uint32_t)H * 4u + 4u;
            // the loads return raw 32-bit words: reinterpret, do not convert
            if (has_g) {
                gv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(args.g + tok, span), voff, 0, 0));
                if (GATE_SUM && CH == 128 && half == 1) {
                    // the second half's gate starts from the first half's total
                    g_first = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                        make_rsrc(args.g + tok, span), (uint32_t)lane * (uint32_t)H * 4u, 0, 0));
                }
            }
            if (args.beta != nullptr) {
                bv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(args.beta + tok, span), voff, 0, 0));
            }
        }

        // ---- a2: K fragments, all loads issued up front (rows >= L read as 0).
        // Each load instruction reads 64 bytes of 16 rows; the next k-step reads
        // the other half of the same 128-byte lines, so these loads are not
        // marked streaming (the lines must survive in L2 until then).  The
        // scheduling barrier keeps every load ahead of the first MFMA, so the
        // whole tile is in flight at once.
        // (the bytes beyond K, when K is below the template's K, read as zeros
        // or are zeroed before the Gram: load_key_frags, mask_key_tail)
        if constexpr (SPLIT != 0) key_offsets();
        load_key_frags<K, kInBytes>(frag, k_rsrc, key_voff, 0, args.k_head_bytes);
        __builtin_amdgcn_sched_barrier(0);

        // ---- gate from per-token log-decays (kkt_solve_gate_cumsum): the
        // gate is their running sum from the chunk's first row, an inclusive
        // scan across the wave (rows >= L hold 0 and come after every valid
        // row).  It needs only g, the first load issued, so it runs while the
        // K tile is still arriving.
        if (GATE_SUM && has_g) {
            gv = wave_prefix_sum(gv, lane);
            if constexpr (CH == 128) {
                // 128-token chunks: the second half adds the first half's
                // total; the A21 waves write the summed gate of both halves
                if (half == 1) {
                    const float total = __shfl(wave_prefix_sum(g_first, lane), kWave - 1, kWave);
                    gv = total + gv;
                }
            }
            g_sum = gv;  // written to g_out after the tile's rows (below)
        }

        // ---- a5, first part: the row and column scales of the epilogue.
        // They need only g and beta, the first loads issued, so they are
        // formed and put in LDS while the K tile is still arriving.
        bool factored = true;
        if (has_g) {
            // reference: row 0's gate (always a valid row), so the factors of
            // rows < L do not depend on L.  If every valid row is within 25 of
            // it, every pair differs by at most 50 (the clamp cannot bind) and
            // every factor lies in [e^-25, e^25].
            const float gref = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, gv)));
            factored = __all(!valid || fabsf(gv - gref) <= 0.5f * kGateClamp);
            if (factored) {
                const float d = gv - gref;
                lds.row_scale[lane] = valid ? bv * __expf(d) : 0.0f;
                lds.col_scale[lane] = valid ? __expf(-d) : 0.0f;
            } else {
                lds.row_scale[lane] = valid ? bv : 0.0f;
                lds.gate[lane] = valid ? gv : 0.0f;
            }
        } else {
            lds.row_scale[lane] = valid ? bv : 0.0f;
        }
        wave_lds_sync();

        mask_key_tail<K, kInBytes>(frag, 0, q, args.k_head_bytes);
        // ---- a4: Gram blocks.  Block (i, j): lane (q, n=m) holds rows 16i + 4q + r, column 16j + n.
        f32x4 S[4][4];
        bool epilogue_done = false;  // a5 already applied, block row by block row
        if constexpr (IN == Elt::F32) {
            // fp32 keys: k-outer, each pair of fragments split once for all
            // ten blocks (the split parts of one pair are all that is live)
            static_assert(kSteps % 2 == 0, "fragment pairs");
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int j = 0; j <= i; ++j) S[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
#pragma unroll
            for (int s = 0; s < kSteps; s += 2) {
                Bf16x3 sp[4];
#pragma unroll
                for (int bi = 0; bi < 4; ++bi) sp[bi] = split_bf16x3(frag[bi][s], frag[bi][s + 1]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
#pragma unroll
                    for (int j = 0; j <= i; ++j) S[i][j] = gram_bf16x3(sp[i], sp[j], S[i][j]);
                }
            }
        } else {
            auto gram = [&](int i, int j) -> f32x4 {
                f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int s = 0; s < kSteps; ++s) acc = gram_step<IN>(frag[i][s], frag[j][s], acc);
                return acc;
            };
            if constexpr (!SHARE && SPLIT == 0) {
                // With a factored gate or none, each block row is scaled
                // right after its Gram blocks (the same operations as a5
                // below, bit for bit), so rows 0..2 are done while row 3's
                // keys may still be arriving.  Same box, us:
                // (2,16384,32,128) 75.1 -> 73.2, its gate-sum form 77.7 ->
                // 75.0, kkt_scaled_dot 97.9 -> 97.0; (1,8192,8,128) 7.0-7.1
                // -> 7.0.  Not in the two-wave tiles of small grids (32
                // tiles 4.39 -> 4.73) nor with the shared key image, whose
                // write and barrier come first.
                if (!has_g || factored) {
                    constexpr float kOff0 = (MODE == Mode::ScaledDot) ? 1.0f : -1.0f;
                    float cc[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) cc[j] = has_g ? lds.col_scale[16 * j + m] : 1.0f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
#pragma unroll
                        for (int j = 0; j <= i; ++j) S[i][j] = gram(i, j);
                        const f32x4 rr = *reinterpret_cast<const f32x4*>(&lds.row_scale[16 * i + 4 * q]);
#pragma unroll
                        for (int j = 0; j <= i; ++j) A[i][j] = (rr * S[i][j]) * (j < i ? kOff0 * cc[j] : cc[j]);
                        if constexpr (MODE == Mode::Fused) {
                            // the diagonal block to LDS for the solve, as below
                            // (4096 tiles 19.83 -> 19.63 us)
                            f32x4 v;
#pragma unroll
                            for (int r = 0; r < 4; ++r) v[r] = (4 * q + r > m) ? -A[i][i][r] : 0.0f;
                            *reinterpret_cast<f32x4*>(&blk[i][m][4 * q]) = v;
                        }
                    }
                    epilogue_done = true;
                    diag_in_lds = (MODE == Mode::Fused);
                }
            }
            if (!epilogue_done) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
#pragma unroll
                    for (int j = 0; j <= i; ++j) S[i][j] = gram(i, j);
                }
            }
        }
        if constexpr (SHARE) {
            if (half == 0) {
                // rows >= L hold the zeros their out-of-range loads returned
#pragma unroll
                for (int bi = 0; bi < 4; ++bi) {
#pragma unroll
                    for (int s = 0; s < kSteps; ++s) ex->kimg[bi][s][lane] = frag[bi][s];
                }
            }
            __syncthreads();  // the first half's key fragments are in LDS
        }

        // ---- a5: epilogue (the scales are in LDS already)
        // (for the solve, the off-diagonal blocks are formed negated: a
        // negated factor negates the rounded product exactly; A itself, for
        // kkt_scaled_dot, keeps its sign)
        constexpr float kOff = (MODE == Mode::ScaledDot) ? 1.0f : -1.0f;
        if (epilogue_done) {
            // (16-bit keys without the shared image: done with the Gram)
        } else if (!has_g) {
            // A = beta_i S (rows >= L have beta 0 and zero keys)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4 rr = *reinterpret_cast<const f32x4*>(&lds.row_scale[16 * i + 4 * q]);
#pragma unroll
                for (int j = 0; j <= i; ++j) A[i][j] = (j < i ? kOff * rr : rr) * S[i][j];
            }
        } else if (factored) {
            // A = (r_i S) c_j: both factors are zero outside the chunk's L rows
            float cc[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) cc[j] = lds.col_scale[16 * j + m];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4 rr = *reinterpret_cast<const f32x4*>(&lds.row_scale[16 * i + 4 * q]);
#pragma unroll
                for (int j = 0; j <= i; ++j) A[i][j] = (rr * S[i][j]) * (j < i ? kOff * cc[j] : cc[j]);
            }
        } else {
            // A = beta_i S exp(clamp(g_i - g_j)); the clamp bounds the gate, so
            // zero keys and zero beta outside the chunk still give 0
            float gc[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) gc[j] = lds.gate[16 * j + m];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4 rr = *reinterpret_cast<const f32x4*>(&lds.row_scale[16 * i + 4 * q]);
                const f32x4 gr = *reinterpret_cast<const f32x4*>(&lds.gate[16 * i + 4 * q]);
#pragma unroll
                for (int j = 0; j <= i; ++j) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float d = fminf(fmaxf(gr[r] - gc[j], -kGateClamp), kGateClamp);
                        A[i][j][r] = (j < i ? kOff * rr[r] : rr[r]) * (S[i][j][r] * __expf(d));
                    }
                }
            }
        }
    }  // A from k, g, beta
    // The output's buffer resource, spanning exactly rows 0 .. L-1 of the
    // chunk (first needed by the stores below).
    const __amdgpu_buffer_rsrc_t o_rsrc = make_rsrc(
        static_cast<char*>(args.out) + tok * (int64_t)(CH * kOutBytes),
        (uint32_t)(L - 1) * args.o_row_bytes + CH * kOutBytes);

    // ---- a8 helper: stage one 16-row block row and write full output rows
    // (rows >= L fall outside o_rsrc and are dropped)
    const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
    auto store_block_row = [&](int i, f32x4 b0, f32x4 b1, f32x4 b2, f32x4 b3) {
        wave_lds_sync();  // earlier reads of the area are done
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
                const f32x4 v = *reinterpret_cast<const f32x4*>(&lds.stage[rr][c4]);
                const uint32_t voff = (row_base + (uint32_t)(16 * i + rr)) * args.o_row_bytes + (col_base + c4) * 4;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), o_rsrc, voff, 0, kNonTemporal);
                if (CH == 128 && half == 0) {  // columns 64..127 of the first half's rows
                    __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, o_rsrc, voff + 64 * 4, 0, kNonTemporal);
                }
            }
        } else {
            // 8 lanes per 128-byte row, 8 rows per pass
            const int rsub = lane / 8, c8 = (lane % 8) * 8;
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const int rr = 8 * it + rsub;
                const f32x4 v0 = *reinterpret_cast<const f32x4*>(&lds.stage[rr][c8]);
                const f32x4 v1 = *reinterpret_cast<const f32x4*>(&lds.stage[rr][c8 + 4]);
                u32x4 p;
                p[0] = pack2<OUT>(v0[0], v0[1]);
                p[1] = pack2<OUT>(v0[2], v0[3]);
                p[2] = pack2<OUT>(v1[0], v1[1]);
                p[3] = pack2<OUT>(v1[2], v1[3]);
                const uint32_t voff = (row_base + (uint32_t)(16 * i + rr)) * args.o_row_bytes + (col_base + c8) * 2;
                __builtin_amdgcn_raw_buffer_store_b128(p, o_rsrc, voff, 0, kNonTemporal);
                if (CH == 128 && half == 0) {
                    __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, o_rsrc, voff + 64 * 2, 0, kNonTemporal);
                }
            }
        }
    };

    // One 128-byte line of each of the 16 rows of block row i of a 64-token
    // chunk with fp32 output: columns 32 hl .. 32 hl + 31 from the blocks b0
    // and b1 (8 lanes per line, 8 rows per pass).
    // (called only where OUT is F32 and CH is 64)
    auto store_row_line = [&](int i, int hl, f32x4 b0, f32x4 b1) {
        wave_lds_sync();  // earlier reads of the area are done
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            lds.stage[4 * q + r][0 + m] = b0[r];
            lds.stage[4 * q + r][16 + m] = b1[r];
        }
        wave_lds_sync();
        const int rsub = lane / 8, c4 = (lane % 8) * 4;
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int rr = 8 * it + rsub;
            const f32x4 v = *reinterpret_cast<const f32x4*>(&lds.stage[rr][c4]);
            const uint32_t voff = (row_base + (uint32_t)(16 * i + rr)) * args.o_row_bytes + (col_base + 32 * hl + c4) * 4;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), o_rsrc, voff, 0, kNonTemporal);
        }
    };
    (void)store_row_line;
    // Columns 32..63 of block row i (0 or 1) of a 64-token chunk with fp32
    // output: all zeros, stored straight from registers.
    auto store_zero_lines = [&](int i) {
        const int rsub = lane / 8, c4 = (lane % 8) * 4;
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int rr = 8 * it + rsub;
            const uint32_t voff = (row_base + (uint32_t)(16 * i + rr)) * args.o_row_bytes + (col_base + 32 + c4) * 4;
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, o_rsrc, voff, 0, kNonTemporal);
        }
    };
    (void)store_zero_lines;

    if constexpr (MODE == Mode::ScaledDot) {
        // ---- A itself: strict lower triangle of every chunk, zeros elsewhere
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) A[i][i][r] = (4 * q + r > m) ? A[i][i][r] : 0.0f;
        }
        store_block_row(0, A[0][0], zero4, zero4, zero4);
        store_block_row(1, A[1][0], A[1][1], zero4, zero4);
        store_block_row(2, A[2][0], A[2][1], A[2][2], zero4);
        store_block_row(3, A[3][0], A[3][1], A[3][2], A[3][3]);
        return;
    }

    // strict lower triangle inside the diagonal blocks, negated and stored
    // transposed (blk[d][col][row]): lane (q, n) holds rows 4q..4q+3 of
    // column n, one 16-byte write, and each lane of the solve below reads its
    // column as one contiguous row
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (!owns(i) || diag_in_lds) continue;
        f32x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (4 * q + r > m) ? -A[i][i][r] : 0.0f;
        *reinterpret_cast<f32x4*>(&blk[i][m][4 * q]) = v;
    }
    wave_lds_sync();

    // ---- a6: X_dd = (I + A_dd)^{-1}; lane (d = lane / 16, c = lane % 16)
    // computes column c of X_dd by right-looking forward substitution: once
    // x[p] is final, every later row takes its term, acc[r] -= A[r][p] x[p].
    // acc[r] starts at [r == c]; rows above c stay exactly 0.  Each lane
    // reads its own column of -A_dd once; the element A[r][p] that step p
    // needs is row r of lane p's column, which a DPP row broadcast
    // (row_newbcast:p, lane p of each 16-lane row to the whole row: the 16
    // lanes of one block) feeds straight into the FMA.  A step's updates are
    // independent, so the dependent chain is one FMA per row, and no step
    // waits on LDS.
    if constexpr (SPLIT != 2) {
        const int d = lane / 16;
        const int c = lane % 16;
        float col[16];  // -A_dd[r][c]; zero for r <= c
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(&blk[d][c][4 * u]);
            col[4 * u + 0] = v[0];
            col[4 * u + 1] = v[1];
            col[4 * u + 2] = v[2];
            col[4 * u + 3] = v[3];
        }
        float acc[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = (r == c) ? 1.0f : 0.0f;
        // Step p: acc[r] = fma(-A[r][p], acc[p], acc[r]) for r = p+1 .. 15,
        // one v_fmac_f32 with the broadcast on its first operand per row.
        // One statement per step; its leading s_nop covers the two wait
        // states a DPP instruction needs after a VALU write of a VGPR it
        // reads (the previous step's results, or any copy the compiler
        // makes of an input), and inside a step no instruction reads what
        // another one writes.
#define KKT_BCAST_FMAC(r, p) "v_fmac_f32_dpp %[a" #r "], %[c" #r "], %[x] row_newbcast:" #p " row_mask:0xf bank_mask:0xf\n"
#define KKT_ACC(r) [a##r] "+v"(acc[r])
#define KKT_COL(r) [c##r] "v"(col[r])
        asm("s_nop 1\n" KKT_BCAST_FMAC(1, 0) KKT_BCAST_FMAC(2, 0) KKT_BCAST_FMAC(3, 0) KKT_BCAST_FMAC(4, 0) KKT_BCAST_FMAC(5, 0) KKT_BCAST_FMAC(6, 0) KKT_BCAST_FMAC(7, 0) KKT_BCAST_FMAC(8, 0) KKT_BCAST_FMAC(9, 0) KKT_BCAST_FMAC(10, 0) KKT_BCAST_FMAC(11, 0) KKT_BCAST_FMAC(12, 0) KKT_BCAST_FMAC(13, 0) KKT_BCAST_FMAC(14, 0) KKT_BCAST_FMAC(15, 0)
            : KKT_ACC(1), KKT_ACC(2), KKT_ACC(3), KKT_ACC(4), KKT_ACC(5), KKT_ACC(6), KKT_ACC(7), KKT_ACC(8), KKT_ACC(9), KKT_ACC(10), KKT_ACC(11), KKT_ACC(12), KKT_ACC(13), KKT_ACC(14), KKT_ACC(15)
            : KKT_COL(1), KKT_COL(2), KKT_COL(3), KKT_COL(4), KKT_COL(5), KKT_COL(6), KKT_COL(7), KKT_COL(8), KKT_COL(9), KKT_COL(10), KKT_COL(11), KKT_COL(12), KKT_COL(13), KKT_COL(14), KKT_COL(15), [x] "v"(acc[0]));
        asm("s_nop 1\n" KKT_BCAST_FMAC(2, 1) KKT_BCAST_FMAC(3, 1) KKT_BCAST_FMAC(4, 1) KKT_BCAST_FMAC(5, 1) KKT_BCAST_FMAC(6, 1) KKT_BCAST_FMAC(7, 1) KKT_BCAST_FMAC(8, 1) KKT_BCAST_FMAC(9, 1) KKT_BCAST_FMAC(10, 1) KKT_BCAST_FMAC(11, 1) KKT_BCAST_FMAC(12, 1) KKT_BCAST_FMAC(13, 1) KKT_BCAST_FMAC(14, 1) KKT_BCAST_FMAC(15, 1)
            : KKT_ACC(2), KKT_ACC(3), KKT_ACC(4), KKT_ACC(5), KKT_ACC(6), KKT_ACC(7), KKT_ACC(8), KKT_ACC(9), KKT_ACC(10), KKT_ACC(11), KKT_ACC(12), KKT_ACC(13), KKT_ACC(14), KKT_ACC(15)
            : KKT_COL(2), KKT_COL(3), KKT_COL(4), KKT_COL(5), KKT_COL(6), KKT_COL(7), KKT_COL(8), KKT_COL(9), KKT_COL(10), KKT_COL(11), KKT_COL(12), KKT_COL(13), KKT_COL(14), KKT_COL(15), [x] "v"(acc[1]));
        asm("s_nop 1\n" KKT_BCAST_FMAC(3, 2) KKT_BCAST_FMAC(4, 2) KKT_BCAST_FMAC(5, 2) KKT_BCAST_FMAC(6, 2) KKT_BCAST_FMAC(7, 2) KKT_BCAST_FMAC(8, 2) KKT_BCAST_FMAC(9, 2) KKT_BCAST_FMAC(10, 2) KKT_BCAST_FMAC(11, 2) KKT_BCAST_FMAC(12, 2) KKT_BCAST_FMAC(13, 2) KKT_BCAST_FMAC(14, 2) KKT_BCAST_FMAC(15, 2)
            : KKT_ACC(3), KKT_ACC(4), KKT_ACC(5), KKT_ACC(6), KKT_ACC(7), KKT_ACC(8), KKT_ACC(9), KKT_ACC(10), KKT_ACC(11), KKT_ACC(12), KKT_ACC(13), KKT_ACC(14), KKT_ACC(15)
            : KKT_COL(3), KKT_COL(4), KKT_COL(5), KKT_COL(6), KKT_COL(7), KKT_COL(8), KKT_COL(9), KKT_COL(10), KKT_COL(11), KKT_COL(12), KKT_COL(13), KKT_COL(14), KKT_COL(15), [x] "v"(acc[2]));
        asm("s_nop 1\n" KKT_BCAST_FMAC(4, 3) KKT_BCAST_FMAC(5, 3) KKT_BCAST_FMAC(6, 3) KKT_BCAST_FMAC(7, 3) KKT_BCAST_FMAC(8, 3) KKT_BCAST_FMAC(9, 3) KKT_BCAST_FMAC(10, 3) KKT_BCAST_FMAC(11, 3) KKT_BCAST_FMAC(12, 3) KKT_BCAST_FMAC(13, 3) KKT_BCAST_FMAC(14, 3) KKT_BCAST_FMAC(15, 3)
            : KKT_ACC(4), KKT_ACC(5), KKT_ACC(6), KKT_ACC(7), KKT_ACC(8), KKT_ACC(9), KKT_ACC(10), KKT_ACC(11), KKT_ACC(12), KKT_ACC(13), KKT_ACC(14), KKT_ACC(15)
            : KKT_COL(4), KKT_COL(5), KKT_COL(6), KKT_COL(7), KKT_COL(8), KKT_COL(9), KKT_COL(10), KKT_COL(11), KKT_COL(12), KKT_COL(13), KKT_COL(14), KKT_COL(15), [x] "v"(acc[3]));
        asm("s_nop 1\n" KKT_BCAST_FMAC(5, 4) KKT_BCAST_FMAC(6, 4) KKT_BCAST_FMAC(7, 4) KKT_BCAST_FMAC(8, 4) KKT_BCAST_FMAC(9, 4) KKT_BCAST_FMAC(10, 4) KKT_BCAST_FMAC(11, 4) KKT_BCAST_FMAC(12, 4) KKT_BCAST_FMAC(13, 4) KKT_BCAST_FMAC(14, 4) KKT_BCAST_FMAC(15, 4)
            : KKT_ACC(5), KKT_ACC(6), KKT_ACC(7), KKT_ACC(8), KKT_ACC(9), KKT_ACC(10), KKT_ACC(11), KKT_ACC(12), KKT_ACC(13), KKT_ACC(14), KKT_ACC(15)
            : KKT_COL(5), KKT_COL(6), KKT_COL(7), KKT_COL(8), KKT_COL(9), KKT_COL(10), KKT_COL(11), KKT_COL(12), KKT_COL(13), KKT_COL(14), KKT_COL(15), [x] "v"(acc[4]));
        asm("s_nop 1\n" KKT_BCAST_FMAC(6, 5) KKT_BCAST_FMAC(7, 5) KKT_BCAST_FMAC(8, 5) KKT_BCAST_FMAC(9, 5) KKT_BCAST_FMAC(10, 5) KKT_BCAST_FMAC(11, 5) KKT_BCAST_FMAC(12, 5) KKT_BCAST_FMAC(13, 5) KKT_BCAST_FMAC(14, 5) KKT_BCAST_FMAC(15, 5)
            : KKT_ACC(6), KKT_ACC(7), KKT_ACC(8), KKT_ACC(9), KKT_ACC(10), KKT_ACC(11), KKT_ACC(12), KKT_ACC(13), KKT_ACC(14), KKT_ACC(15)
            : KKT_COL(6), KKT_COL(7), KKT_COL(8), KKT_COL(9), KKT_COL(10), KKT_COL(11), KKT_COL(12), KKT_COL(13), KKT_COL(14), KKT_COL(15), [x] "v"(acc[5]));
        asm("s_nop 1\n" KKT_BCAST_FMAC(7, 6) KKT_BCAST_FMAC(8, 6) KKT_BCAST_FMAC(9, 6) KKT_BCAST_FMAC(10, 6) KKT_BCAST_FMAC(11, 6) KKT_BCAST_FMAC(12, 6) KKT_BCAST_FMAC(13, 6) KKT_BCAST_FMAC(14, 6) KKT_BCAST_FMAC(15, 6)
            : KKT_ACC(7), KKT_ACC(8), KKT_ACC(9), KKT_ACC(10), KKT_ACC(11), KKT_ACC(12), KKT_ACC(13), KKT_ACC(14), KKT_ACC(15)
            : KKT_COL(7), KKT_COL(8), KKT_COL(9), KKT_COL(10), KKT_COL(11), KKT_COL(12), KKT_COL(13), KKT_COL(14), KKT_COL(15), [x] "v"(acc[6]));
        asm("s_nop 1\n" KKT_BCAST_FMAC(8, 7) KKT_BCAST_FMAC(9, 7) KKT_BCAST_FMAC(10, 7) KKT_BCAST_FMAC(11, 7) KKT_BCAST_FMAC(12, 7) KKT_BCAST_FMAC(13, 7) KKT_BCAST_FMAC(14, 7) KKT_BCAST_FMAC(15, 7)
            : KKT_ACC(8), KKT_ACC(9), KKT_ACC(10), KKT_ACC(11), KKT_ACC(12), KKT_ACC(13), KKT_ACC(14), KKT_ACC(15)
            : KKT_COL(8), KKT_COL(9), KKT_COL(10), KKT_COL(11), KKT_COL(12), KKT_COL(13), KKT_COL(14), KKT_COL(15), [x] "v"(acc[7]));
        asm("s_nop 1\n" KKT_BCAST_FMAC(9, 8) KKT_BCAST_FMAC(10, 8) KKT_BCAST_FMAC(11, 8) KKT_BCAST_FMAC(12, 8) KKT_BCAST_FMAC(13, 8) KKT_BCAST_FMAC(14, 8) KKT_BCAST_FMAC(15, 8)
            : KKT_ACC(9), KKT_ACC(10), KKT_ACC(11), KKT_ACC(12), KKT_ACC(13), KKT_ACC(14), KKT_ACC(15)
            : KKT_COL(9), KKT_COL(10), KKT_COL(11), KKT_COL(12), KKT_COL(13), KKT_COL(14), KKT_COL(15), [x] "v"(acc[8]));
        asm("s_nop 1\n" KKT_BCAST_FMAC(10, 9) KKT_BCAST_FMAC(11, 9) KKT_BCAST_FMAC(12, 9) KKT_BCAST_FMAC(13, 9) KKT_BCAST_FMAC(14, 9) KKT_BCAST_FMAC(15, 9)
            : KKT_ACC(10), KKT_ACC(11), KKT_ACC(12), KKT_ACC(13), KKT_ACC(14), KKT_ACC(15)
            : KKT_COL(10), KKT_COL(11), KKT_COL(12), KKT_COL(13), KKT_COL(14), KKT_COL(15), [x] "v"(acc[9]));
        asm("s_nop 1\n" KKT_BCAST_FMAC(11, 10) KKT_BCAST_FMAC(12, 10) KKT_BCAST_FMAC(13, 10) KKT_BCAST_FMAC(14, 10) KKT_BCAST_FMAC(15, 10)
            : KKT_ACC(11), KKT_ACC(12), KKT_ACC(13), KKT_ACC(14), KKT_ACC(15)
            : KKT_COL(11), KKT_COL(12), KKT_COL(13), KKT_COL(14), KKT_COL(15), [x] "v"(acc[10]));
        asm("s_nop 1\n" KKT_BCAST_FMAC(12, 11) KKT_BCAST_FMAC(13, 11) KKT_BCAST_FMAC(14, 11) KKT_BCAST_FMAC(15, 11)
            : KKT_ACC(12), KKT_ACC(13), KKT_ACC(14), KKT_ACC(15)
            : KKT_COL(12), KKT_COL(13), KKT_COL(14), KKT_COL(15), [x] "v"(acc[11]));
        asm("s_nop 1\n" KKT_BCAST_FMAC(13, 12) KKT_BCAST_FMAC(14, 12) KKT_BCAST_FMAC(15, 12)
            : KKT_ACC(13), KKT_ACC(14), KKT_ACC(15)
            : KKT_COL(13), KKT_COL(14), KKT_COL(15), [x] "v"(acc[12]));
        asm("s_nop 1\n" KKT_BCAST_FMAC(14, 13) KKT_BCAST_FMAC(15, 13)
            : KKT_ACC(14), KKT_ACC(15)
            : KKT_COL(14), KKT_COL(15), [x] "v"(acc[13]));
        asm("s_nop 1\n" KKT_BCAST_FMAC(15, 14)
            : KKT_ACC(15)
            : KKT_COL(15), [x] "v"(acc[14]));
#undef KKT_BCAST_FMAC
#undef KKT_ACC
#undef KKT_COL
        wave_lds_sync();  // every read of A_dd precedes the overwrite with X_dd
        // X_dd stored transposed as well: column c is contiguous
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const f32x4 v = {acc[4 * u], acc[4 * u + 1], acc[4 * u + 2], acc[4 * u + 3]};
            *reinterpret_cast<f32x4*>(&blk[d][c][4 * u]) = v;
        }
    }
    wave_lds_sync();
    if constexpr (SPLIT != 0) __syncthreads();  // split tile: all four diagonal inverses are in blk
    if constexpr (GATE_SUM && SPLIT == 1) {
        // both waves loaded the decays before this barrier
        if (args.g != nullptr && args.g_out != nullptr) {
            const uint32_t span = (uint32_t)(L - 1) * (uint32_t)H * 4u + 4u;
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, g_sum), make_rsrc(args.g_out + tok, span),
                                                  (uint32_t)lane * (uint32_t)H * 4u, 0, 0);
        }
    }

    // X_dd in both operand layouts (blk[d][col][row] = X_dd[row][col]):
    //   xa[d]: lane (q, m) holds X_dd[m][4q .. 4q+3]   (left operand)
    //   xd[d]: lane (q, n) holds X_dd[4q .. 4q+3][n]   (right operand / result layout)
    // (the solve of a given A negates xa instead of its loaded A blocks: see
    // below)
    constexpr float kXaSign = (MODE == Mode::SolveTril) ? -1.0f : 1.0f;
    f32x4 xa[4], xd[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        xd[d] = *reinterpret_cast<const f32x4*>(&blk[d][m][4 * q]);
#pragma unroll
        for (int r = 0; r < 4; ++r) xa[d][r] = kXaSign * blk[d][4 * q + r][m];
    }

    // ---- a7: merge.  wt_ik = -(X_ii A_ik)^T: the off-diagonal blocks of A
    // arrive negated from the epilogue (its column factor carries the sign),
    // and the solve of a given A negates xa (negating it as each element of
    // A loads cost that kernel 0.5 us of 6.3 on (1,8192,8,128)); a negated
    // factor negates each product exactly, so both give the same bits.  The
    // result layout of wt is the left-operand layout of -W_ik, and every
    // X_ij = -sum_k W_ik X_kj is a plain accumulation (the same value, bit
    // for bit, as 0 - sum: negating every product negates the rounded sum,
    // and an all-zero sum stays +0.0 from the +0.0 start).
    if constexpr (SPLIT == 1) {
        // block rows 0..2; X10 and X21 go to the other wave before the
        // second barrier, X20 before the third
        store_block_row(0, xd[0], zero4, zero4, zero4);
        const f32x4 wt10 = mm16(A[1][0], xa[1], zero4);
        const f32x4 wt20 = mm16(A[2][0], xa[2], zero4);
        const f32x4 wt21 = mm16(A[2][1], xa[2], zero4);
        const f32x4 x10 = mm16(wt10, xd[0], zero4);
        const f32x4 x21 = mm16(wt21, xd[1], zero4);
        const f32x4 p20 = mm16(wt20, xd[0], zero4);
        xchg[0][lane] = x10;
        xchg[1][lane] = x21;
        __syncthreads();
        store_block_row(1, x10, xd[1], zero4, zero4);
        const f32x4 x20 = mm16(wt21, x10, p20);
        xchg[2][lane] = x20;
        __syncthreads();
        store_block_row(2, x20, x21, xd[2], zero4);
        return;
    } else if constexpr (SPLIT == 2) {
        // block row 3
        const f32x4 wt30 = mm16(A[3][0], xa[3], zero4);
        const f32x4 wt31 = mm16(A[3][1], xa[3], zero4);
        const f32x4 wt32 = mm16(A[3][2], xa[3], zero4);
        const f32x4 x32 = mm16(wt32, xd[2], zero4);
        const f32x4 p31 = mm16(wt31, xd[1], zero4);
        f32x4 p30 = mm16(wt30, xd[0], zero4);
        __syncthreads();
        const f32x4 x10 = xchg[0][lane];
        const f32x4 x21 = xchg[1][lane];
        p30 = mm16(wt31, x10, p30);
        const f32x4 x31 = mm16(wt32, x21, p31);
        __syncthreads();
        const f32x4 x20 = xchg[2][lane];
        const f32x4 x30 = mm16(wt32, x20, p30);
        store_block_row(3, x30, x31, x32, xd[3]);
        return;
    }

    if constexpr (GATE_SUM && CH == 64) {
        // The summed gate, one 4-byte word per lane into 64 cache lines that
        // the tiles of the other heads write too, when each wave writes its
        // own words: issued with the first output lines, before the W
        // products, so that it drains during the merge.  Issued right after
        // the scan, while the key tile was still arriving, these stores cost
        // 0.9 us of 8.5 on (1,8192,8,128); after the last rows, bf16 output,
        // 7.22 vs 7.13 us here (same box).
        if (args.g != nullptr && args.g_out != nullptr && !args.gate_gather) {
            const uint32_t span = (uint32_t)(L - 1) * (uint32_t)H * 4u + 4u;
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, g_sum),
                                                  make_rsrc(args.g_out + tok, span),
                                                  (uint32_t)lane * (uint32_t)H * 4u, 0, 0);
        }
    }
    if constexpr (OUT == Elt::F32 && CH == 64) {
        // fp32 lines that need only the diagonal inverses (below): issued
        // before the six W products, whose MFMAs then run while these
        // stores drain (the LDS barriers of a staged store bound the
        // compiler's scheduling).  Same box, us: (1,8192,8,128) 6.93-7.03
        // -> 6.84-6.93, its gate-sum form 7.29-7.38 -> 7.17-7.21, 512 tiles
        // 5.65-5.69 -> 5.60-5.62; 2048 and 4096 tiles about 1% slower,
        // 16384 tiles unchanged.
        store_row_line(0, 0, xd[0], zero4);
        store_zero_lines(0);
        store_row_line(2, 1, xd[2], zero4);
    }
    const f32x4 wt10 = mm16(A[1][0], xa[1], zero4);
    const f32x4 wt20 = mm16(A[2][0], xa[2], zero4);
    const f32x4 wt21 = mm16(A[2][1], xa[2], zero4);
    const f32x4 wt30 = mm16(A[3][0], xa[3], zero4);
    const f32x4 wt31 = mm16(A[3][1], xa[3], zero4);
    const f32x4 wt32 = mm16(A[3][2], xa[3], zero4);

    {
        // The blocks are formed in the result layout and staged through LDS,
        // so that every store instruction writes whole 128-byte lines (4 rows
        // of 256 bytes, or 8 of 128; fp32 line by line below).  Stored straight
        // from registers, each instruction writes a 64- or 32-byte piece of
        // 16 rows, twice or four times the cache lines per instruction: that
        // measured slower in the store phase on the bench workload and 1.6
        // times slower overall on the (2,16384,32,128) workload.  With
        // 128-token chunks this half's blocks also go to the rest of the
        // workgroup.
        // The partial products that do not wait on this level's results are
        // issued before each store, so the MFMA pipe works through them while
        // the store's LDS and memory instructions execute.
        f32x4 x10, x21, x32, x20, x31, x30;
        if constexpr (OUT == Elt::F32 && CH == 64) {
            // fp32 rows of 64-token chunks are two 128-byte lines (columns
            // 0..31, 32..63), and each line goes out once its two blocks are
            // final: the right half of block row 2 (X22, zeros) right after
            // the diagonal inverses, that of block row 3 (X32, X33) after the
            // first merge level, the left halves after the second and third.
            // After the last product 2 KB of the tile's 16 remain to be
            // written instead of 8.  Same box, us: (1,8192,8,128) 7.47-7.53
            // -> 7.32-7.38, 512 tiles 6.25-6.36 -> 5.99-6.12, 4096 tiles
            // 24.64-24.76 -> 24.28-24.35; fp32 keys unchanged.  The all-zero
            // right halves of block rows 0 and 1 skip the LDS staging
            // (another box: 7.12-7.20 -> 7.03-7.06, 4096 tiles 19.94-20.04 ->
            // 19.75-19.81; stored right after the key loads instead, they
            // cost 0.1-0.2 us).  In the two-wave tiles of small grids the
            // same line stores took longer: 32 tiles 4.38 -> 4.70 us, 250
            // tiles with fp32 output 4.85 -> 5.07 us.
            // (block row 0 and the right half of block row 2 went out
            // before the W products, above)
            x10 = mm16(wt10, xd[0], zero4);
            x21 = mm16(wt21, xd[1], zero4);
            x32 = mm16(wt32, xd[2], zero4);
            const f32x4 p20 = mm16(wt20, xd[0], zero4);
            const f32x4 p31 = mm16(wt31, xd[1], zero4);
            f32x4 p30 = mm16(wt30, xd[0], zero4);
            store_row_line(1, 0, x10, xd[1]);
            store_zero_lines(1);
            store_row_line(3, 1, x32, xd[3]);

            x20 = mm16(wt21, x10, p20);
            x31 = mm16(wt32, x21, p31);
            p30 = mm16(wt31, x10, p30);
            store_row_line(2, 0, x20, x21);

            x30 = mm16(wt32, x20, p30);
            store_row_line(3, 0, x30, x31);
        } else {
            store_block_row(0, xd[0], zero4, zero4, zero4);
            x10 = mm16(wt10, xd[0], zero4);
            x21 = mm16(wt21, xd[1], zero4);
            x32 = mm16(wt32, xd[2], zero4);
            const f32x4 p20 = mm16(wt20, xd[0], zero4);
            const f32x4 p31 = mm16(wt31, xd[1], zero4);
            f32x4 p30 = mm16(wt30, xd[0], zero4);
            store_block_row(1, x10, xd[1], zero4, zero4);

            x20 = mm16(wt21, x10, p20);
            x31 = mm16(wt32, x21, p31);
            p30 = mm16(wt31, x10, p30);
            store_block_row(2, x20, x21, xd[2], zero4);

            x30 = mm16(wt32, x20, p30);
            store_block_row(3, x30, x31, x32, xd[3]);
        }

        if constexpr (GATE_SUM && CH == 64) {
            // The workgroup's gathered store of the summed gate (run_tile)
            // takes this wave's sums from row_scale, no longer read here.
            if (args.g != nullptr && args.g_out != nullptr && args.gate_gather) {
                wave_lds_sync();
                lds.row_scale[lane] = g_sum;
            }
        }

        if constexpr (CH == 128) {
            __syncthreads();  // end of the first phase: the exchange area overlaps its areas
            // hand the block to the workgroup: X11 as result-layout register
            // images, X22 row-major (each lane of a reader then takes 4
            // consecutive entries of one row, a left operand, in one load)
            const f32x4 blocks[10] = {xd[0], x10, xd[1], x20, x21, xd[2], x30, x31, x32, xd[3]};
            if (half == 0) {
#pragma unroll
                for (int b = 0; b < 10; ++b) ex->cross.x11[b][lane] = blocks[b];
            } else {
#pragma unroll
                for (int b = 0; b < 10; ++b) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) ex->x22[b][4 * q + r][m] = blocks[b][r];
                }
            }
        }
    }
}


// One 64-token chunk per wave, four waves per workgroup.
template <Mode MODE, Elt IN, Elt OUT, int K, bool GATE_SUM = false>
__device__ __forceinline__ void run_tile(const KernelArgs& args, WaveLds* lds_all)
{
    const int lane = threadIdx.x % kWave;
    // wave-uniform values are pinned to scalar registers so that the buffer
    // resources built from them are scalar too
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t tile_id = workgroup_order(args) * (uint32_t)args.tile_waves + wave;
    if (tile_id >= (uint32_t)args.n_tiles) return;  // wave-uniform

    // ---- a1: tile map
    const int H = args.H;
    const uint32_t chunk = fast_div(tile_id, args.div_H);
    const int h = (int)(tile_id - chunk * (uint32_t)H);
    const Tile tile = chunk_tile<kChunk>(args, chunk, lane);
    if (tile.len <= 0) return;  // wave-uniform
    chunk_rows<MODE, IN, OUT, K, GATE_SUM, kChunk>(args, lds_all[wave], lds_all[wave].blk, nullptr, lane,
                                                   tile.row0 * H + h, tile.len, 0, nullptr);
    if constexpr (GATE_SUM && MODE == Mode::Fused) {
        // Large grids of fixed-length rows with H a multiple of 4: the four
        // tiles of this workgroup are heads h - wave .. h - wave + 3 of one
        // chunk (every one valid), and their summed gates of a token are 16
        // contiguous bytes, written by one lane: a quarter of the strided
        // write requests.  (2,16384,32,128): 80.9 -> 77.8 us; on
        // (1,8192,8,128), one tile per SIMD, the barrier cost 0.2 us, so
        // there each wave writes its own words.
        if (args.gate_gather) {
            __syncthreads();  // every wave's row_scale holds its summed gate
            const int t = 16 * wave + lane;
            if (lane < 16 && t < tile.len) {
                const f32x4 v = {lds_all[0].row_scale[t], lds_all[1].row_scale[t], lds_all[2].row_scale[t],
                                 lds_all[3].row_scale[t]};
                const uint32_t span = (uint32_t)(tile.len - 1) * (uint32_t)H * 4u + 16u;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v),
                                                       make_rsrc(args.g_out + tile.row0 * H + (h - wave), span),
                                                       (uint32_t)t * (uint32_t)H * 4u, 0, 0);
            }
        }
    }
}

// LDS of a 64-token tile split over two waves: their own gate arrays and
// store stages, the shared diagonal blocks and the exchanged X10, X21, X20.
struct SplitLds {
    WaveLds wave[2];
    float blk[4][16][kBlockLd];
    f32x4 xchg[3][kWave];
};

// One 64-token chunk per two-wave workgroup (the fused op, or the solve of
// a given A, on small grids, where a tile's latency, not the chip's
// throughput, sets the time).  Both waves sum the gate of a GATE_SUM tile,
// with the same scan.
template <Mode MODE, Elt IN, Elt OUT, int K, bool GATE_SUM = false>
__device__ __forceinline__ void run_split_tile(const KernelArgs& args, SplitLds& lds)
{
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t tile_id = workgroup_order(args);
    if (tile_id >= (uint32_t)args.n_tiles) return;  // workgroup-uniform
    const int H = args.H;
    const uint32_t chunk = fast_div(tile_id, args.div_H);
    const int h = (int)(tile_id - chunk * (uint32_t)H);
    const Tile tile = chunk_tile<kChunk>(args, chunk, lane);
    if (tile.len <= 0) return;  // workgroup-uniform
    const int64_t tok = tile.row0 * H + h;
    if (wave == 0) {
        chunk_rows<MODE, IN, OUT, K, GATE_SUM, kChunk, false, 1>(args, lds.wave[0], lds.blk, lds.xchg, lane, tok,
                                                                 tile.len, 0, nullptr);
    } else {
        chunk_rows<MODE, IN, OUT, K, GATE_SUM, kChunk, false, 2>(args, lds.wave[1], lds.blk, lds.xchg, lane, tok,
                                                                 tile.len, 0, nullptr);
    }
}

// 128-token chunks: the 64x64 block A21 of A (rows 64..127, columns 0..63)
// for two of its four 16-row block rows (w2 = 0: rows 64..95, 1: rows
// 96..127), left in the workgroup's LDS as left-operand-layout images.
// A21[i][j] = beta_i (k_i . k_j) exp(clamp(g_i - g_j)), formed like the
// diagonal blocks: as a row and a column factor around the Gram when the
// chunk's gates lie within half the clamp of its first row's, else with a
// clamped exponential per element.
struct CrossIn {
    float g_lo;  // gate of first-half row `lane` (a column of A21)
    float g_hi;  // gate of second-half row 64 + lane
    float b_hi;  // beta of second-half row 64 + lane
};

__device__ __forceinline__ CrossIn cross_gate_beta(const KernelArgs& args, int lane, int64_t tok, int L)
{
    const int H = args.H;
    CrossIn c{0.0f, 0.0f, 1.0f};  // rows >= L read 0
    const uint32_t span = (uint32_t)(L - 1) * (uint32_t)H * 4u + 4u;
    const uint32_t lo = (uint32_t)lane * (uint32_t)H * 4u, hi = (64u + (uint32_t)lane) * (uint32_t)H * 4u;
    if (args.g != nullptr) {
        const __amdgpu_buffer_rsrc_t g_rsrc = make_rsrc(args.g + tok, span);
        c.g_lo = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(g_rsrc, lo, 0, 0));
        c.g_hi = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(g_rsrc, hi, 0, 0));
    }
    if (args.beta != nullptr) {
        c.b_hi = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(args.beta + tok, span), hi, 0, 0));
    }
    return c;
}

// Gate-sum kernel, 128-token chunks: the loaded per-token decays of the two
// halves become the chunk's summed gate (the second half starts from the
// first half's total), bit for bit as the halves' own waves form it.
__device__ __forceinline__ void cross_gate_sum(CrossIn& c, int lane)
{
    const float lo = wave_prefix_sum(c.g_lo, lane);
    const float total = __shfl(lo, kWave - 1, kWave);
    c.g_lo = lo;
    c.g_hi = total + wave_prefix_sum(c.g_hi, lane);
}

// acc[bi][bj]: S21 block (2 w2 + bi, bj) in left-operand layout, i.e. lane
// (q, m) holds S21[m][4q + r]: second-half row 32 w2 + 16 bi + m, first-half
// column 16 bj + 4q + r.  Turned into the A21 blocks in place.
__device__ __forceinline__ void cross_scale(const KernelArgs& args, GateLds& lds, int lane, int w2, int L,
                                            const CrossIn& in, f32x4 (&acc)[2][4])
{
    const int q = lane / 16;
    const int m = lane % 16;
    const bool has_g = args.g != nullptr;
    const bool valid_lo = lane < L, valid_hi = 64 + lane < L;
    // Factored gate, as in the 64-row epilogue: with every valid gate of the
    // chunk within 25 of row 0's, A21_ij = (r_i S21_ij) c_j with
    // r_i = beta_i exp(g_i - g_0) and c_j = exp(g_0 - g_j) (the clamp
    // cannot bind); otherwise each element takes its clamped exponential.
    bool factored = false;
    if (has_g) {
        const float gref = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, in.g_lo)));
        factored = __all((!valid_lo || fabsf(in.g_lo - gref) <= 0.5f * kGateClamp) &&
                         (!valid_hi || fabsf(in.g_hi - gref) <= 0.5f * kGateClamp));
        if (factored) {
            lds.row_scale[lane] = valid_hi ? in.b_hi * __expf(in.g_hi - gref) : 0.0f;
            lds.col_scale[lane] = valid_lo ? __expf(gref - in.g_lo) : 0.0f;
        } else {
            lds.row_scale[lane] = in.b_hi;
            lds.gate[lane] = in.g_hi;
            lds.col_scale[lane] = in.g_lo;
        }
    } else {
        lds.row_scale[lane] = in.b_hi;
    }
    wave_lds_sync();
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
        const int row = 32 * w2 + 16 * bi + m;
        const float br = lds.row_scale[row];
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
            f32x4 a;
            if (!has_g) {
                a = br * acc[bi][bj];
            } else if (factored) {
                const f32x4 cc = *reinterpret_cast<const f32x4*>(&lds.col_scale[16 * bj + 4 * q]);
                a = (br * acc[bi][bj]) * cc;
            } else {
                const float gr = lds.gate[row];
                const f32x4 gc = *reinterpret_cast<const f32x4*>(&lds.col_scale[16 * bj + 4 * q]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float d = fminf(fmaxf(gr - gc[r], -kGateClamp), kGateClamp);
                    a[r] = br * (acc[bi][bj][r] * __expf(d));
                }
            }
            acc[bi][bj] = a;
        }
    }
}

__device__ __forceinline__ void cross_store(Chunk128Lds& ex, int lane, int w2, const f32x4 (&a21)[2][4])
{
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) ex.cross.a21[4 * (2 * w2 + bi) + bj][lane] = a21[bi][bj];
    }
}

// S21 blocks from key fragments: gram_step(first-half fragment, second-half
// fragment) gives K1_j K2_i^T in result layout, which is S21_ij in
// left-operand layout.
template <Elt IN, int P>
__device__ __forceinline__ void cross_gram(const u32x4 (&fr)[2][P], const u32x4 (&fc)[4][P], f32x4 (&acc)[2][4])
{
    if constexpr (IN == Elt::F32) {
        static_assert(P % 2 == 0, "fragment pairs");
#pragma unroll
        for (int s = 0; s < P; s += 2) {
            Bf16x3 r[2], c[4];
#pragma unroll
            for (int bi = 0; bi < 2; ++bi) r[bi] = split_bf16x3(fr[bi][s], fr[bi][s + 1]);
#pragma unroll
            for (int bj = 0; bj < 4; ++bj) c[bj] = split_bf16x3(fc[bj][s], fc[bj][s + 1]);
#pragma unroll
            for (int bi = 0; bi < 2; ++bi) {
#pragma unroll
                for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = gram_bf16x3(c[bj], r[bi], acc[bi][bj]);
            }
        }
    } else {
#pragma unroll
        for (int bi = 0; bi < 2; ++bi) {
#pragma unroll
            for (int bj = 0; bj < 4; ++bj) {
#pragma unroll
                for (int s = 0; s < P; ++s) acc[bi][bj] = gram_step<IN>(fc[bj][s], fr[bi][s], acc[bi][bj]);
            }
        }
    }
}

// A21 blocks (the rows of w2; scaled, in registers) with the keys read from
// global memory in passes of at most 4 fragments per row (head dimensions
// whose key fragments do not fit the LDS image).
template <Elt IN, int K, bool GATE_SUM>
__device__ __forceinline__ void cross_block_rows(const KernelArgs& args, GateLds& lds, int lane, int64_t tok, int L,
                                                 int w2, f32x4 (&acc)[2][4], CrossIn& in)
{
    constexpr int kInBytes = EltInfo<IN>::bytes;
    constexpr int kElemsPer16B = 16 / kInBytes;
    constexpr int kSteps = K / (4 * kElemsPer16B);
    constexpr int kPass = kSteps < 4 ? kSteps : 4;  // fragments per row and pass (register budget)
    static_assert(kSteps % kPass == 0, "whole passes");
    const int q = lane / 16;
    const int m = lane % 16;
    const __amdgpu_buffer_rsrc_t k_rsrc = make_rsrc(
        static_cast<const char*>(args.k) + tok * (int64_t)args.k_head_bytes,
        (uint32_t)(L - 1) * args.k_row_bytes + args.k_head_bytes);
    in = cross_gate_beta(args, lane, tok, L);
    if (GATE_SUM && args.g != nullptr) cross_gate_sum(in, lane);
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int p0 = 0; p0 < kSteps; p0 += kPass) {
        u32x4 fr[2][kPass], fc[4][kPass];
        uint32_t vr[2], vc[4];
#pragma unroll
        for (int bi = 0; bi < 2; ++bi) vr[bi] = (uint32_t)(64 + 32 * w2 + 16 * bi + m) * args.k_row_bytes + q * 16;
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) vc[bj] = (uint32_t)(16 * bj + m) * args.k_row_bytes + q * 16;
        load_key_frags<K, kInBytes>(fr, k_rsrc, vr, p0, args.k_head_bytes);
        load_key_frags<K, kInBytes>(fc, k_rsrc, vc, p0, args.k_head_bytes);
        __builtin_amdgcn_sched_barrier(0);
        mask_key_tail<K, kInBytes>(fr, p0, q, args.k_head_bytes);
        mask_key_tail<K, kInBytes>(fc, p0, q, args.k_head_bytes);
        cross_gram<IN, kPass>(fr, fc, acc);
        __builtin_amdgcn_sched_barrier(0);
    }
    cross_scale(args, lds, lane, w2, L, in, acc);
}

// The one-wave-per-tile kernels size their LDS at launch: one WaveLds per
// wave of the workgroup (1 or 4), so that one-wave workgroups take 5.9 KB.
__device__ __forceinline__ WaveLds* tile_lds()
{
    extern __shared__ __align__(16) char lds_raw[];
    return reinterpret_cast<WaveLds*>(lds_raw);
}

// One kernel per entry point, so that profiles name the operation.
template <Elt IN, Elt OUT, int K>
__global__ __launch_bounds__(kWave * kWavesPerGroup)
void kkt_solve_kernel(KKT_KERNEL_PARAMS)
{
    KKT_KERNEL_ARGS;
    WaveLds* lds_all = tile_lds();
    run_tile<Mode::Fused, IN, OUT, K>(args, lds_all);
}

// The fused op with each 64-token tile split over a two-wave workgroup.
template <Elt IN, Elt OUT, int K>
__global__ __launch_bounds__(kWave * 2)
void kkt_solve_split_kernel(KKT_KERNEL_PARAMS)
{
    KKT_KERNEL_ARGS;
    __shared__ SplitLds lds;
    run_split_tile<Mode::Fused, IN, OUT, K>(args, lds);
}

template <Elt IN, Elt OUT, int K>
__global__ __launch_bounds__(kWave * kWavesPerGroup)
void kkt_solve_gate_cumsum_kernel(KKT_KERNEL_PARAMS)
{
    KKT_KERNEL_ARGS;
    WaveLds* lds_all = tile_lds();
    run_tile<Mode::Fused, IN, OUT, K, true>(args, lds_all);
}

template <Elt IN, Elt OUT, int K>
__global__ __launch_bounds__(kWave * 2)
void kkt_solve_gate_cumsum_split_kernel(KKT_KERNEL_PARAMS)
{
    KKT_KERNEL_ARGS;
    __shared__ SplitLds lds;
    run_split_tile<Mode::Fused, IN, OUT, K, true>(args, lds);
}

template <Elt IN, int K>
__global__ __launch_bounds__(kWave * kWavesPerGroup)
void kkt_scaled_dot_kernel(KKT_KERNEL_PARAMS)
{
    KKT_KERNEL_ARGS;
    WaveLds* lds_all = tile_lds();
    run_tile<Mode::ScaledDot, IN, Elt::F32, K>(args, lds_all);
}

// (the input-type and K arguments of run_tile are unused in this mode)
template <Elt OUT>
__global__ __launch_bounds__(kWave * kWavesPerGroup)
void kkt_solve_tril_kernel(KKT_KERNEL_PARAMS)
{
    KKT_KERNEL_ARGS;
    WaveLds* lds_all = tile_lds();
    run_tile<Mode::SolveTril, Elt::F32, OUT, 64>(args, lds_all);
}

template <Elt OUT>
__global__ __launch_bounds__(kWave * 2)
void kkt_solve_tril_split_kernel(KKT_KERNEL_PARAMS)
{
    KKT_KERNEL_ARGS;
    __shared__ SplitLds lds;
    run_split_tile<Mode::SolveTril, Elt::F32, OUT, 64>(args, lds);
}

// 128-token chunks (the GDR case page's chunk size), one workgroup per
// (chunk, head).  With X11 = (I + A11)^{-1}, X22 = (I + A22)^{-1} for the two
// 64-row halves, the inverse is [[X11, 0], [X21, X22]] with
// X21 = -X22 (A21 X11):
//   waves 0, 1: a2-a8 on their half (X11, X22 and their output columns);
//   waves 2, 3: A21, two block rows each;
//   then P = A21 X11 (wave i: block row i), X21 = -X22 P (wave j: block
//   column j), X21 staged in LDS and stored as 256/128-byte row pieces.
// How the key tile reaches the waves (STAGE):
//   kKeysShared: waves 0 and 1 load their halves into registers as the
//                64-token pipeline does; after its Gram, wave 0 copies the
//                first half's fragments to LDS, where waves 2 and 3 read them
//                (their own 32 second-half rows they read after that barrier,
//                from L2).  Waves 0 and 1 wait for no other wave before their
//                Gram, and waves 2 and 3 are idle until then anyway.  The LDS
//                image holds at most 4 k-steps (16-bit keys with K <= 128,
//                fp32 keys with K = 64).
//   kKeysGlobal: (larger K) every wave loads the key rows it needs; waves 2
//                and 3 read the first half and their own rows again, in
//                passes of 4 k-steps.
enum KeyStage { kKeysGlobal = 0, kKeysShared = 1 };

template <Elt IN, Elt OUT, int K, int STAGE, bool GATE_SUM>
__global__ __launch_bounds__(kWave * kWavesPerGroup)
// (shared 16-bit keys: at most 128 VGPRs, so that registers, like the 39 KB
// of LDS, leave room for four workgroups per CU; split fp32 keys need more)
__attribute__((amdgpu_waves_per_eu(STAGE == kKeysShared && IN != Elt::F32 ? 4 : 1)))
void kkt_solve128_kernel(KKT_KERNEL_PARAMS)
{
    KKT_KERNEL_ARGS;
    constexpr int kOutBytes = EltInfo<OUT>::bytes;
    __shared__ Chunk128Lds ex;
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int q = lane / 16;
    const int m = lane % 16;
    const uint32_t tile_id = workgroup_order(args);
    if (tile_id >= (uint32_t)args.n_tiles) return;  // workgroup-uniform
    const int H = args.H;
    const uint32_t chunk = fast_div(tile_id, args.div_H);
    const int h = (int)(tile_id - chunk * (uint32_t)H);
    const Tile tile = chunk_tile<2 * kChunk>(args, chunk, lane);
    if (tile.len <= 0) return;  // workgroup-uniform
    const int L = tile.len;
    const int64_t tok = tile.row0 * H + h;

    constexpr int kInBytes = EltInfo<IN>::bytes;
    constexpr int kSteps = K / (4 * (16 / kInBytes));
    static_assert(STAGE == kKeysGlobal || kSteps <= 4, "the LDS key image holds at most 4 k-steps");
    float gsum_lo = 0.0f, gsum_hi = 0.0f;  // GATE_SUM: wave 2's summed gate, stored last
    (void)gsum_lo;
    (void)gsum_hi;
    if (wave < 2) {
        chunk_rows<Mode::Fused, IN, OUT, K, GATE_SUM, 2 * kChunk, STAGE == kKeysShared>(
            args, ex.half[wave], ex.half[wave].blk, nullptr, lane, tok, L, wave, &ex);
    } else {
        const int w2 = wave - 2;
        f32x4 acc[2][4];
        CrossIn cin;
        if constexpr (STAGE == kKeysShared) {
            // the first half's fragments from wave 0 via LDS; the own rows
            // (64 + 32 w2 ..) from memory, but only after the barrier: wave 1
            // has fetched them by then (L2 hits), and issued at the start
            // they would queue in front of the loads of waves 0 and 1
            const __amdgpu_buffer_rsrc_t k_rsrc = make_rsrc(
                static_cast<const char*>(args.k) + tok * (int64_t)args.k_head_bytes,
                (uint32_t)(L - 1) * args.k_row_bytes + args.k_head_bytes);
            cin = cross_gate_beta(args, lane, tok, L);
            if (GATE_SUM && args.g != nullptr) cross_gate_sum(cin, lane);
#pragma unroll
            for (int bi = 0; bi < 2; ++bi) {
#pragma unroll
                for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
            __syncthreads();  // the first half's key fragments are in LDS
            u32x4 fr[2][kSteps];
            uint32_t vr[2];
#pragma unroll
            for (int bi = 0; bi < 2; ++bi) vr[bi] = (uint32_t)(64 + 32 * w2 + 16 * bi + m) * args.k_row_bytes + q * 16;
            load_key_frags<K, kInBytes>(fr, k_rsrc, vr, 0, args.k_head_bytes);
            mask_key_tail<K, kInBytes>(fr, 0, q, args.k_head_bytes);
            constexpr int kPer = (IN == Elt::F32) ? 2 : 1;  // fragments per Gram step
#pragma unroll
            for (int s = 0; s < kSteps; s += kPer) {
                u32x4 fc[4][kPer], fs[2][kPer];
#pragma unroll
                for (int e = 0; e < kPer; ++e) {
#pragma unroll
                    for (int bj = 0; bj < 4; ++bj) fc[bj][e] = ex.kimg[bj][s + e][lane];
                    fs[0][e] = fr[0][s + e];
                    fs[1][e] = fr[1][s + e];
                }
                cross_gram<IN, kPer>(fs, fc, acc);
            }
            cross_scale(args, ex.cross_gate[w2], lane, w2, L, cin, acc);
        } else {
            cross_block_rows<IN, K, GATE_SUM>(args, ex.cross_gate[w2], lane, tok, L, w2, acc, cin);
        }
        __syncthreads();  // end of the first phase: the exchange area overlaps its areas
        cross_store(ex, lane, w2, acc);
        if constexpr (GATE_SUM) {
            gsum_lo = cin.g_lo;
            gsum_hi = cin.g_hi;
        }
    }
    __syncthreads();

    const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
    // P = A21 X11, block row i = wave: P_ij = sum_{k=j..3} A21_ik X11_kj
    {
        const int i = wave;
        f32x4 a[4], p[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) a[k] = ex.cross.a21[4 * i + k][lane];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            p[j] = zero4;
#pragma unroll
            for (int k = j; k < 4; ++k) p[j] = mm16(a[k], ex.cross.x11[tri(k, j)][lane], p[j]);
        }
        wave_lds_sync();  // this wave's reads of its A21 row precede the overwrite
#pragma unroll
        for (int j = 0; j < 4; ++j) ex.cross.a21[4 * i + j][lane] = p[j];
    }
    __syncthreads();

    // X21 = -X22 P, block column j = wave: X21_ij = -sum_{k=0..i} X22_ik P_kj
    f32x4 x21[4];
    {
        const int j = wave;
        f32x4 pc[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) pc[k] = ex.cross.a21[4 * k + j][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x4 sum = zero4;
#pragma unroll
            for (int k = 0; k <= i; ++k) {
                // X22_ik in left-operand layout: row m, columns 4q .. 4q+3
                const f32x4 xa = *reinterpret_cast<const f32x4*>(&ex.x22[tri(i, k)][m][4 * q]);
                sum = mm16(xa, pc[k], sum);
            }
            x21[i] = zero4 - sum;
        }
    }
    __syncthreads();  // every read of the exchange area is done: X21 may overwrite it

    // stage block column j = wave of X21 as rows, then store rows 64 + 16 wave ..
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) ex.x21[16 * i + 4 * q + r][16 * wave + m] = x21[i][r];
    }
    __syncthreads();
    const __amdgpu_buffer_rsrc_t o_rsrc = make_rsrc(
        static_cast<char*>(args.out) + tok * (int64_t)(2 * kChunk * kOutBytes),
        (uint32_t)(L - 1) * args.o_row_bytes + 2 * kChunk * kOutBytes);
    if constexpr (OUT == Elt::F32) {
        const int rsub = lane / 16, c4 = (lane % 16) * 4;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int rr = 16 * wave + 4 * it + rsub;
            const f32x4 v = *reinterpret_cast<const f32x4*>(&ex.x21[rr][c4]);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), o_rsrc,
                                                   (uint32_t)(64 + rr) * args.o_row_bytes + c4 * 4, 0, kNonTemporal);
        }
    } else {
        const int rsub = lane / 8, c8 = (lane % 8) * 8;
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int rr = 16 * wave + 8 * it + rsub;
            const f32x4 v0 = *reinterpret_cast<const f32x4*>(&ex.x21[rr][c8]);
            const f32x4 v1 = *reinterpret_cast<const f32x4*>(&ex.x21[rr][c8 + 4]);
            u32x4 p;
            p[0] = pack2<OUT>(v0[0], v0[1]);
            p[1] = pack2<OUT>(v0[2], v0[3]);
            p[2] = pack2<OUT>(v1[0], v1[1]);
            p[3] = pack2<OUT>(v1[2], v1[3]);
            __builtin_amdgcn_raw_buffer_store_b128(p, o_rsrc, (uint32_t)(64 + rr) * args.o_row_bytes + c8 * 2, 0,
                                                   kNonTemporal);
        }
    }
    if constexpr (GATE_SUM) {
        // the summed gate of both halves, after the rows (strided 4-byte
        // words: see the 64-token tile; every wave has read its decays long
        // before, so g_out may alias them)
        if (wave == 2 && args.g != nullptr && args.g_out != nullptr) {
            const uint32_t span = (uint32_t)(L - 1) * (uint32_t)H * 4u + 4u;
            const __amdgpu_buffer_rsrc_t go = make_rsrc(args.g_out + tok, span);
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, gsum_lo), go,
                                                  (uint32_t)lane * (uint32_t)H * 4u, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, gsum_hi), go,
                                                  (64u + (uint32_t)lane) * (uint32_t)H * 4u, 0, 0);
        }
    }
}

// ---------------------------------------------------------------- host side
thread_local std::string g_last_error;

kkt_status_t fail(kkt_status_t st, const std::string& msg)
{
    g_last_error = msg;
    return st;
}

// Per-device "is gfx950" cache: 0 unknown, 1 yes, 2 no.  Lock-free: two
// threads that find it unknown both query the device and store the same
// value.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

kkt_status_t check_device()
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(KKT_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(KKT_ERR_UNSUPPORTED, "device index out of range");
    int ok = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (ok == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return fail(KKT_ERR_HIP, std::string("hipGetDeviceProperties: ") + hipGetErrorString(e));
        ok = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_arch_ok[dev].store(ok, std::memory_order_relaxed);
    }
    if (ok != 1) return fail(KKT_ERR_UNSUPPORTED, "device is not gfx950 (MI355X); this library is built for gfx950 only");
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

// The kernels are built for K = 64, 128 and 256; any other K runs in the
// next one up, with the key bytes beyond it read or zeroed as 0 (k_step_rsrc,
// mask_key_tail).
int64_t k_bucket(int64_t K) { return K <= 64 ? 64 : (K <= 128 ? 128 : 256); }

// waves: the workgroup size in waves; the one-wave-per-tile kernels take
// a.tile_waves (their default), the others name theirs
using KernelFn = void (*)(uint64_t, uint64_t, uint64_t, uint64_t, uint64_t, uint32_t, uint32_t, uint32_t, uint32_t,
                          KernelArgs);

// The log2 of a power of two v >= 1.
uint32_t log2_exact(uint32_t v)
{
    uint32_t l = 0;
    while ((1u << l) < v) ++l;
    return l;
}

// An address with a field in its top 16 bits (KKT_KERNEL_PARAMS).
uint64_t with_field(const void* p, uint32_t field)
{
    return reinterpret_cast<uint64_t>(p) | ((uint64_t)(field & 0xffffu) << 48);
}

hipError_t launch(KernelFn kernel, const KernelArgs& a, hipStream_t stream, int waves = 0)
{
    // (the one-wave-per-tile kernels take one WaveLds per wave as dynamic LDS)
    const size_t lds_bytes = (waves > 0) ? 0 : (size_t)a.tile_waves * sizeof(WaveLds);
    // the preloaded fields (see KKT_KERNEL_PARAMS); setup() checks that they fit
    const uint32_t tw = (uint32_t)a.tile_waves;
    const uint32_t o_head_bytes = a.o_row_bytes / (uint32_t)a.H;
    if ((tw != 1 && tw != 4) || a.n_groups != (((uint32_t)a.n_tiles + tw - 1u) >> (tw >> 1)) ||
        a.k_head_bytes % 16u != 0 || a.k_head_bytes / 16u > 127u || o_head_bytes < 128u || o_head_bytes > 512u) {
        return hipErrorInvalidConfiguration;  // not reached: setup() makes them so
    }
    const uint32_t fk = (uint32_t)a.xcd_order | ((uint32_t)a.log2_group_run << 2) | (tw << 7) |
                        (a.div_H.shift << 10) | ((uint32_t)a.packed << 15);
    const uint32_t fo = a.div_chunks.shift | ((log2_exact(o_head_bytes) - 7u) << 5) | ((a.k_head_bytes / 16u) << 7) |
                        ((uint32_t)a.gate_gather << 14);
    hipLaunchKernelGGL(kernel, dim3(a.n_groups), dim3(kWave * (waves > 0 ? waves : a.tile_waves)), lds_bytes, stream,
                       with_field(a.k, fk), with_field(a.g, a.div_chunks.magic & 0xffffu),
                       with_field(a.beta, a.div_chunks.magic >> 16), with_field(a.out, fo), with_field(a.g_out, 0),
                       (uint32_t)a.n_tiles, (uint32_t)a.H, a.div_H.magic, (uint32_t)a.T, a);
    return hipGetLastError();
}

template <Elt IN, Elt OUT, bool GATE_SUM>
hipError_t launch_fused(int64_t K, const KernelArgs& a, hipStream_t stream)
{
    K = k_bucket(K);
    if constexpr (GATE_SUM) {
        if (a.split_tiles) {
            switch (K) {
            case 64: return launch(kkt_solve_gate_cumsum_split_kernel<IN, OUT, 64>, a, stream, 2);
            case 128: return launch(kkt_solve_gate_cumsum_split_kernel<IN, OUT, 128>, a, stream, 2);
            default: return launch(kkt_solve_gate_cumsum_split_kernel<IN, OUT, 256>, a, stream, 2);
            }
        }
        switch (K) {
        case 64: return launch(kkt_solve_gate_cumsum_kernel<IN, OUT, 64>, a, stream);
        case 128: return launch(kkt_solve_gate_cumsum_kernel<IN, OUT, 128>, a, stream);
        default: return launch(kkt_solve_gate_cumsum_kernel<IN, OUT, 256>, a, stream);
        }
    } else if (a.split_tiles) {
        switch (K) {
        case 64: return launch(kkt_solve_split_kernel<IN, OUT, 64>, a, stream, 2);
        case 128: return launch(kkt_solve_split_kernel<IN, OUT, 128>, a, stream, 2);
        default: return launch(kkt_solve_split_kernel<IN, OUT, 256>, a, stream, 2);
        }
    } else {
        switch (K) {
        case 64: return launch(kkt_solve_kernel<IN, OUT, 64>, a, stream);
        case 128: return launch(kkt_solve_kernel<IN, OUT, 128>, a, stream);
        default: return launch(kkt_solve_kernel<IN, OUT, 256>, a, stream);
        }
    }
}

template <Elt IN, Elt OUT, int K, bool GATE_SUM>
hipError_t launch_fused128_k(const KernelArgs& a, hipStream_t stream)
{
    constexpr int kSteps = K / (4 * (16 / EltInfo<IN>::bytes));
    return launch(kkt_solve128_kernel<IN, OUT, K, (kSteps <= 4) ? kKeysShared : kKeysGlobal, GATE_SUM>, a, stream,
                  kWavesPerGroup);
}

template <Elt IN, Elt OUT, bool GATE_SUM>
hipError_t launch_fused128(int64_t K, const KernelArgs& a, hipStream_t stream)
{
    K = k_bucket(K);
    switch (K) {
    case 64: return launch_fused128_k<IN, OUT, 64, GATE_SUM>(a, stream);
    case 128: return launch_fused128_k<IN, OUT, 128, GATE_SUM>(a, stream);
    default: return launch_fused128_k<IN, OUT, 256, GATE_SUM>(a, stream);
    }
}

template <Elt IN, bool GATE_SUM = false>
hipError_t launch_fused_out(kkt_dtype_t od, int64_t K, int64_t chunk, const KernelArgs& a, hipStream_t stream)
{
    if (chunk == 2 * kChunk) {
        switch (od) {
        case KKT_DTYPE_F32: return launch_fused128<IN, Elt::F32, GATE_SUM>(K, a, stream);
        case KKT_DTYPE_BF16: return launch_fused128<IN, Elt::BF16, GATE_SUM>(K, a, stream);
        default: return launch_fused128<IN, Elt::F16, GATE_SUM>(K, a, stream);
        }
    }
    switch (od) {
    case KKT_DTYPE_F32: return launch_fused<IN, Elt::F32, GATE_SUM>(K, a, stream);
    case KKT_DTYPE_BF16: return launch_fused<IN, Elt::BF16, GATE_SUM>(K, a, stream);
    default: return launch_fused<IN, Elt::F16, GATE_SUM>(K, a, stream);
    }
}

template <Elt IN>
hipError_t launch_scaled_dot(int64_t K, const KernelArgs& a, hipStream_t stream)
{
    K = k_bucket(K);
    switch (K) {
    case 64: return launch(kkt_scaled_dot_kernel<IN, 64>, a, stream);
    case 128: return launch(kkt_scaled_dot_kernel<IN, 128>, a, stream);
    default: return launch(kkt_scaled_dot_kernel<IN, 256>, a, stream);
    }
}

bool valid_dtype(int d) { return d == KKT_DTYPE_F32 || d == KKT_DTYPE_BF16 || d == KKT_DTYPE_F16; }

// The integer a C caller passed for an enum parameter.  C lets any int
// through an enum type; in C++ reading a value outside the enumerators'
// range as the enum type is undefined, so the bytes are read as an int and
// only a validated value is used as the enum.
template <typename E>
int enum_code(const E& e)
{
    static_assert(sizeof(E) == sizeof(int), "C enums are int-sized here");
    int v;
    memcpy(&v, &e, sizeof v);
    return v;
}

int64_t dtype_bytes(kkt_dtype_t d) { return d == KKT_DTYPE_F32 ? 4 : 2; }

// Grids up to this many workgroups use the XCD-contiguous tile order; larger
// ones keep chunks in round-robin order over the XCDs (each XCD's concurrent
// accesses spread over the whole tensor), with all heads of a chunk on one XCD.
constexpr int64_t kRemapMaxGroups = 1024;
// Gate-sum grids of more four-wave workgroups than this gather the summed
// gates of a workgroup's four heads (run_tile).
constexpr int64_t kGateGatherMinGroups = 1024;
#ifndef KKT_LARGE_GRID_ORDER
#define KKT_LARGE_GRID_ORDER kChunkRoundRobin
#endif

// Grids of up to this many 64-token tiles of the fused op (one per CU of
// the chip) run one tile per two-wave workgroup: there the time is a tile's
// latency after its keys arrive, which the split shortens (128 to 256 tiles:
// 21-33% less time), rather than the chip's throughput.  From about 384
// tiles up the split's extra key reads, barriers and second wave per SIMD
// cost as much as the shorter tail saves or more (1024 tiles: 13-25% more
// time).  KKT_SPLIT_TILES overrides the bound (0: never split).
constexpr int64_t kSplitMaxTiles = 256;
constexpr int64_t kSplitAuto = -1;  // KKT_OPTION_SPLIT_MAX_TILES: the library chooses (split_max_tiles)

// Grids that run one tile per wave use workgroups of one wave up to a bound
// (the hardware spreads them over every CU; four-wave workgroups put a small
// grid on a quarter or half of the CUs), of four waves beyond it.  Measured
// one-wave against four-wave workgroups (us, bf16 keys, K = 128): the fused
// op on 512 tiles 6.11-6.14 vs 6.74, on 448 tiles with fp32 keys 9.17-9.19 vs
// 10.34-10.36; the first step of the chain on 256 and 32 tiles 4.15-4.16 vs
// 5.46-5.48 and 3.47-3.48 vs 4.93; at 1024 tiles the fused op 8.22-8.24 vs
// 8.34-8.37, its gate-sum form 8.70-8.74 vs 8.70-8.71, the solve of a given A
// 6.49-6.51 vs 6.44-6.46, the first step of the chain 7.33-7.36 vs
// 6.82-6.87; beyond, four-wave workgroups are faster (16384 tiles: 75.0 vs
// 80.2; 1876: 20.0 vs 21.0-21.4).  Since the key offsets are fixed before
// the g/beta loads, the fused op on 1024 tiles is faster in four-wave
// workgroups (7.43-7.54 vs 7.55-7.66 us, same box), while one-wave ones
// still win on 768 tiles (6.80-6.91 vs 6.85-6.97) and 512 (6.16-6.22 vs
// 6.82-6.86).
constexpr int64_t kWave1GroupTilesFused = 768;   // kkt_solve
constexpr int64_t kWave1GroupTiles = 512;        // the other entry points

// Process-wide options (kkt_set_option).  Their start values come from the
// environment, read once when the library is loaded: KKT_SPLIT_TILES (the
// two-wave bound above) and KKT_VALIDATE=1 (check cu_seqlens on the host).
int64_t env_int(const char* name, int64_t fallback)
{
    const char* v = getenv(name);
    return (v != nullptr && v[0] != '\0') ? strtoll(v, nullptr, 10) : fallback;
}
std::atomic<int64_t> g_split_max_tiles{env_int("KKT_SPLIT_TILES", kSplitAuto)};
std::atomic<int64_t> g_validate_cu_seqlens{env_int("KKT_VALIDATE", 0) == 1 ? 1 : 0};
// The two-wave bound of a call: the option's value, or, by default
// (kSplitAuto), kSplitMaxTiles, except for the fused op with 16-bit keys and
// 16-bit output (one_wave_faster), whose one-wave tiles are faster on every
// grid measured (32-256 tiles: 0.08-0.19 us; with an fp32 output or fp32
// keys the two-wave tiles stay 0.12-0.25 us faster, and so do the gate-sum
// op and the solve of a given A).
int64_t split_max_tiles(bool one_wave_faster)
{
    const int64_t v = g_split_max_tiles.load(std::memory_order_relaxed);
    return (v >= 0) ? v : (one_wave_faster ? 0 : kSplitMaxTiles);
}

FastDiv make_fastdiv(uint32_t d)
{
    uint32_t s = 0;
    while ((2ull << s) <= d) ++s;  // s = floor(log2 d)
    if ((1ull << s) == d) return FastDiv{0u, s};
    const uint64_t magic = ((1ull << (32 + s)) + d - 1) / d;  // ceil(2^(32+s) / d) < 2^32
    return FastDiv{(uint32_t)magic, s};
}

// Checks shared by every entry point and the launch geometry.  in_row_bytes
// and out_row_bytes are the strides between consecutive tokens of one head;
// chunk is 64 (one tile per wave) or 128 (one tile per workgroup).
// Returns KKT_OK with a filled in; makes no HIP call unless the arguments pass.
// Device addresses travel with fields in their top 16 bits (KKT_KERNEL_PARAMS).
bool below_2_48(const void* p) { return (reinterpret_cast<uint64_t>(p) >> 48) == 0; }

kkt_status_t setup(KernelArgs& a, const void* in, const float* g, const float* beta,
                   const int32_t* cu_seqlens, int64_t num_seqs, int64_t B, int64_t T, int64_t H,
                   int64_t in_row_bytes, int64_t out_row_bytes, void* out, hipStream_t stream,
                   int64_t chunk = kChunk, int64_t split_bound = 0, int64_t wave1_group_tiles = 0)
{
    if (in == nullptr || out == nullptr) return fail(KKT_ERR_INVALID_ARGUMENT, "input and output must not be NULL");
    // the kernel moves the row tensors in 16-byte vectors, g / beta / cu_seqlens in 4-byte words
    if ((reinterpret_cast<uintptr_t>(in) & 15u) != 0 || (reinterpret_cast<uintptr_t>(out) & 15u) != 0) {
        return fail(KKT_ERR_INVALID_ARGUMENT, "input and output must be 16-byte aligned");
    }
    if ((reinterpret_cast<uintptr_t>(g) & 3u) != 0 || (reinterpret_cast<uintptr_t>(beta) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) {
        return fail(KKT_ERR_INVALID_ARGUMENT, "g, beta and cu_seqlens must be 4-byte aligned");
    }
    // 32-bit in-tile offsets: the rows of one chunk of one head must span < 2 GiB
    if (chunk * in_row_bytes >= (1LL << 31) || chunk * out_row_bytes >= (1LL << 31)) {
        return fail(KKT_ERR_UNSUPPORTED, "H * K too large for one launch");
    }
    const int64_t chunks_per_row = (T + chunk - 1) / chunk;
    // Packed sequences: at most floor(T/chunk) + num_seqs chunks; surplus tiles exit.
    const int64_t n_chunks = (cu_seqlens == nullptr) ? B * chunks_per_row : T / chunk + num_seqs;
    const int64_t n_tiles = n_chunks * H;
    const bool split = chunk == kChunk && n_tiles <= split_bound;  // two-wave tiles
    // one wave per tile: a workgroup of one wave on grids of up to
    // wave1_group_tiles tiles (spread over every CU), else of four
    const int64_t tiles_per_group =
        (chunk == kChunk && !split) ? ((n_tiles <= wave1_group_tiles) ? 1 : kWavesPerGroup) : 1;
    if (n_tiles >= (1LL << 31) - kWavesPerGroup || num_seqs >= (1LL << 31) - 1) {
        return fail(KKT_ERR_UNSUPPORTED, "problem too large for one launch");
    }
    // T and the bytes of one head's row travel in 32-bit and narrower fields
    // of the preloaded kernel arguments (KKT_KERNEL_PARAMS): a key row of up to
    // 1 KiB, an output row of 128, 256 or 512 bytes
    const int64_t o_head_bytes = out_row_bytes / H;
    if (in_row_bytes % H != 0 || in_row_bytes / H >= 2048 || out_row_bytes % H != 0 ||
        (o_head_bytes != 128 && o_head_bytes != 256 && o_head_bytes != 512)) {
        return fail(KKT_ERR_UNSUPPORTED, "row sizes outside the kernels' range");
    }
    if (T > (int64_t)UINT32_MAX) return fail(KKT_ERR_UNSUPPORTED, "T must be below 2^32 tokens");
    if (!below_2_48(in) || !below_2_48(g) || !below_2_48(beta) || !below_2_48(out)) {
        return fail(KKT_ERR_UNSUPPORTED, "device addresses must lie below 2^48");
    }

    kkt_status_t st = check_device();
    if (st != KKT_OK) return st;
    if (cu_seqlens != nullptr && g_validate_cu_seqlens.load(std::memory_order_relaxed) != 0) {
        st = validate_cu_seqlens(cu_seqlens, num_seqs, T, stream);
        if (st != KKT_OK) return st;
    }

    a.k = in;
    a.g = g;
    a.beta = beta;
    a.cu_seqlens = cu_seqlens;
    a.out = out;
    a.T = T;
    a.num_seqs = (int32_t)num_seqs;
    a.H = (int32_t)H;
    a.div_chunks = make_fastdiv((uint32_t)(chunks_per_row > 0 ? chunks_per_row : 1));
    a.n_tiles = (int32_t)n_tiles;
    a.k_row_bytes = (uint32_t)in_row_bytes;
    a.o_row_bytes = (uint32_t)out_row_bytes;
    const int64_t groups = (n_tiles + tiles_per_group - 1) / tiles_per_group;
    a.n_groups = (uint32_t)groups;
    a.xcd_order = groups <= kRemapMaxGroups ? kContiguous : KKT_LARGE_GRID_ORDER;
    // runs of the largest power of two <= the workgroups per chunk
    const int64_t per_chunk = (H + tiles_per_group - 1) / tiles_per_group;
    int lg = 0;
    while ((2LL << lg) <= per_chunk && lg < 16) ++lg;
    a.log2_group_run = lg;
    a.remap_groups = (uint32_t)((groups >> (lg + 3)) << (lg + 3));
    a.g_out = nullptr;
    a.gate_gather = 0;
    a.packed = (cu_seqlens != nullptr) ? 1 : 0;
    a.split_tiles = split ? 1 : 0;
    a.tile_waves = (int32_t)tiles_per_group;
    a.k_head_bytes = (uint32_t)(in_row_bytes / H);
    a.div_H = make_fastdiv((uint32_t)H);
    return KKT_OK;
}

// Size checks of the entry points that take k.
// K: up to 256, with key rows of whole 16-byte pieces (fp32: a multiple of
// 4; bf16 / f16: a multiple of 8).
kkt_status_t check_k_sizes(int64_t B, int64_t T, int64_t H, int64_t K, int64_t num_seqs, const int32_t* cu_seqlens,
                           int64_t k_elt_bytes)
{
    if (B < 1 || H < 1 || K < 1 || T < 0) return fail(KKT_ERR_INVALID_ARGUMENT, "B, H, K must be >= 1 and T >= 0");
    if (K > 256 || (K * k_elt_bytes) % 16 != 0) {
        return fail(KKT_ERR_UNSUPPORTED, "K must be at most 256 and a multiple of 4 (fp32 keys) or 8 (bf16/f16 keys)");
    }
    if (cu_seqlens != nullptr && (B != 1 || num_seqs < 1)) {
        return fail(KKT_ERR_INVALID_ARGUMENT, "cu_seqlens needs B == 1 and num_seqs >= 1");
    }
    return KKT_OK;
}

}  // namespace

extern "C" kkt_status_t kkt_solve(const void* k, const float* g, const float* beta,
                                  const int32_t* cu_seqlens, int64_t num_seqs,
                                  int64_t B, int64_t T, int64_t H, int64_t K,
                                  int64_t chunk_size, kkt_dtype_t in_dtype_arg, kkt_dtype_t out_dtype_arg,
                                  void* out, hipStream_t stream)
{
    g_last_error.clear();
    // ---- argument checks: no HIP call before they pass
    if (chunk_size != kChunk && chunk_size != 2 * kChunk) return fail(KKT_ERR_UNSUPPORTED, "chunk_size must be 64 or 128");
    if (!valid_dtype(enum_code(in_dtype_arg)) || !valid_dtype(enum_code(out_dtype_arg))) {
        return fail(KKT_ERR_INVALID_ARGUMENT, "unknown dtype");
    }
    const kkt_dtype_t in_dtype = (kkt_dtype_t)enum_code(in_dtype_arg);
    const kkt_dtype_t out_dtype = (kkt_dtype_t)enum_code(out_dtype_arg);
    kkt_status_t st = check_k_sizes(B, T, H, K, num_seqs, cu_seqlens, dtype_bytes(in_dtype));
    if (st != KKT_OK) return st;
    if (T == 0) return KKT_OK;
    KernelArgs a;
    st = setup(a, k, g, beta, cu_seqlens, num_seqs, B, T, H, H * K * dtype_bytes(in_dtype),
               H * chunk_size * dtype_bytes(out_dtype), out, stream, chunk_size,
               split_max_tiles(in_dtype != KKT_DTYPE_F32 && out_dtype != KKT_DTYPE_F32), kWave1GroupTilesFused);
    if (st != KKT_OK) return st;

    hipError_t e;
    switch (in_dtype) {
    case KKT_DTYPE_F32: e = launch_fused_out<Elt::F32>(out_dtype, K, chunk_size, a, stream); break;
    case KKT_DTYPE_BF16: e = launch_fused_out<Elt::BF16>(out_dtype, K, chunk_size, a, stream); break;
    default: e = launch_fused_out<Elt::F16>(out_dtype, K, chunk_size, a, stream); break;
    }
    if (e != hipSuccess) return fail(KKT_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
    return KKT_OK;
}

extern "C" kkt_status_t kkt_solve_gate_cumsum(const void* k, const float* g_decay, const float* beta,
                                              const int32_t* cu_seqlens, int64_t num_seqs,
                                              int64_t B, int64_t T, int64_t H, int64_t K,
                                              int64_t chunk_size, kkt_dtype_t in_dtype_arg, kkt_dtype_t out_dtype_arg,
                                              void* out, float* g_out, hipStream_t stream)
{
    g_last_error.clear();
    if (chunk_size != kChunk && chunk_size != 2 * kChunk) return fail(KKT_ERR_UNSUPPORTED, "chunk_size must be 64 or 128");
    if (!valid_dtype(enum_code(in_dtype_arg)) || !valid_dtype(enum_code(out_dtype_arg))) {
        return fail(KKT_ERR_INVALID_ARGUMENT, "unknown dtype");
    }
    const kkt_dtype_t in_dtype = (kkt_dtype_t)enum_code(in_dtype_arg);
    const kkt_dtype_t out_dtype = (kkt_dtype_t)enum_code(out_dtype_arg);
    kkt_status_t st = check_k_sizes(B, T, H, K, num_seqs, cu_seqlens, dtype_bytes(in_dtype));
    if (st != KKT_OK) return st;
    if (T == 0) return KKT_OK;
    if (g_decay == nullptr) return fail(KKT_ERR_INVALID_ARGUMENT, "g_decay must not be NULL");
    if ((reinterpret_cast<uintptr_t>(g_out) & 3u) != 0) return fail(KKT_ERR_INVALID_ARGUMENT, "g_out must be 4-byte aligned");
    if (!below_2_48(g_out)) return fail(KKT_ERR_UNSUPPORTED, "device addresses must lie below 2^48");
    KernelArgs a;
    st = setup(a, k, g_decay, beta, cu_seqlens, num_seqs, B, T, H, H * K * dtype_bytes(in_dtype),
               H * chunk_size * dtype_bytes(out_dtype), out, stream, chunk_size, split_max_tiles(false),
               kWave1GroupTiles);
    if (st != KKT_OK) return st;
    a.g_out = g_out;
    // four heads' summed gates per 16-byte store (run_tile): only where every
    // four-wave workgroup holds four valid tiles of one chunk, and on grids
    // of more workgroups than run at once on the chip (below that, the
    // barrier it needs lengthens the tiles' tail)
    a.gate_gather = (cu_seqlens == nullptr && chunk_size == kChunk && !a.split_tiles && a.tile_waves == 4 &&
                     H % 4 == 0 && a.n_groups > kGateGatherMinGroups && g_out != nullptr &&
                     (reinterpret_cast<uintptr_t>(g_out) & 15u) == 0) ? 1 : 0;

    hipError_t e;
    switch (in_dtype) {
    case KKT_DTYPE_F32: e = launch_fused_out<Elt::F32, true>(out_dtype, K, chunk_size, a, stream); break;
    case KKT_DTYPE_BF16: e = launch_fused_out<Elt::BF16, true>(out_dtype, K, chunk_size, a, stream); break;
    default: e = launch_fused_out<Elt::F16, true>(out_dtype, K, chunk_size, a, stream); break;
    }
    if (e != hipSuccess) return fail(KKT_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
    return KKT_OK;
}

extern "C" kkt_status_t kkt_scaled_dot(const void* k, const float* g, const float* beta,
                                       const int32_t* cu_seqlens, int64_t num_seqs,
                                       int64_t B, int64_t T, int64_t H, int64_t K,
                                       int64_t chunk_size, kkt_dtype_t in_dtype_arg, float* A, hipStream_t stream)
{
    g_last_error.clear();
    if (chunk_size != kChunk) return fail(KKT_ERR_UNSUPPORTED, "chunk_size must be 64");
    if (!valid_dtype(enum_code(in_dtype_arg))) return fail(KKT_ERR_INVALID_ARGUMENT, "unknown dtype");
    const kkt_dtype_t in_dtype = (kkt_dtype_t)enum_code(in_dtype_arg);
    kkt_status_t st = check_k_sizes(B, T, H, K, num_seqs, cu_seqlens, dtype_bytes(in_dtype));
    if (st != KKT_OK) return st;
    if (T == 0) return KKT_OK;
    KernelArgs a;
    st = setup(a, k, g, beta, cu_seqlens, num_seqs, B, T, H, H * K * dtype_bytes(in_dtype), H * kChunk * 4, A, stream,
               kChunk, 0, kWave1GroupTiles);
    if (st != KKT_OK) return st;

    hipError_t e;
    switch (in_dtype) {
    case KKT_DTYPE_F32: e = launch_scaled_dot<Elt::F32>(K, a, stream); break;
    case KKT_DTYPE_BF16: e = launch_scaled_dot<Elt::BF16>(K, a, stream); break;
    default: e = launch_scaled_dot<Elt::F16>(K, a, stream); break;
    }
    if (e != hipSuccess) return fail(KKT_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
    return KKT_OK;
}

extern "C" kkt_status_t kkt_solve_tril(const float* A, const int32_t* cu_seqlens, int64_t num_seqs,
                                       int64_t B, int64_t T, int64_t H, int64_t chunk_size,
                                       kkt_dtype_t out_dtype_arg, void* out, hipStream_t stream)
{
    g_last_error.clear();
    if (chunk_size != kChunk) return fail(KKT_ERR_UNSUPPORTED, "chunk_size must be 64");
    if (!valid_dtype(enum_code(out_dtype_arg))) return fail(KKT_ERR_INVALID_ARGUMENT, "unknown dtype");
    const kkt_dtype_t out_dtype = (kkt_dtype_t)enum_code(out_dtype_arg);
    if (B < 1 || H < 1 || T < 0) return fail(KKT_ERR_INVALID_ARGUMENT, "B, H must be >= 1 and T >= 0");
    if (cu_seqlens != nullptr && (B != 1 || num_seqs < 1)) {
        return fail(KKT_ERR_INVALID_ARGUMENT, "cu_seqlens needs B == 1 and num_seqs >= 1");
    }
    if (T == 0) return KKT_OK;
    KernelArgs a;
    kkt_status_t st = setup(a, A, nullptr, nullptr, cu_seqlens, num_seqs, B, T, H, H * kChunk * 4,
                            H * kChunk * dtype_bytes(out_dtype), out, stream, kChunk, split_max_tiles(false),
                            kWave1GroupTiles);
    if (st != KKT_OK) return st;

    hipError_t e;
    switch (out_dtype) {
    case KKT_DTYPE_F32:
        e = a.split_tiles ? launch(kkt_solve_tril_split_kernel<Elt::F32>, a, stream, 2)
                          : launch(kkt_solve_tril_kernel<Elt::F32>, a, stream);
        break;
    case KKT_DTYPE_BF16:
        e = a.split_tiles ? launch(kkt_solve_tril_split_kernel<Elt::BF16>, a, stream, 2)
                          : launch(kkt_solve_tril_kernel<Elt::BF16>, a, stream);
        break;
    default:
        e = a.split_tiles ? launch(kkt_solve_tril_split_kernel<Elt::F16>, a, stream, 2)
                          : launch(kkt_solve_tril_kernel<Elt::F16>, a, stream);
        break;
    }
    if (e != hipSuccess) return fail(KKT_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
    return KKT_OK;
}

extern "C" kkt_status_t kkt_set_option(kkt_option_t option_arg, int64_t value)
{
    g_last_error.clear();
    switch (enum_code(option_arg)) {
    case KKT_OPTION_SPLIT_MAX_TILES:
        if (value < kSplitAuto) {
            return fail(KKT_ERR_INVALID_ARGUMENT, "KKT_OPTION_SPLIT_MAX_TILES must be >= 0, or -1 (automatic)");
        }
        g_split_max_tiles.store(value, std::memory_order_relaxed);
        return KKT_OK;
    case KKT_OPTION_VALIDATE_CU_SEQLENS:
        g_validate_cu_seqlens.store(value != 0 ? 1 : 0, std::memory_order_relaxed);
        return KKT_OK;
    }
    return fail(KKT_ERR_INVALID_ARGUMENT, "unknown option");
}

extern "C" int64_t kkt_get_option(kkt_option_t option_arg)
{
    switch (enum_code(option_arg)) {
    case KKT_OPTION_SPLIT_MAX_TILES: return g_split_max_tiles.load(std::memory_order_relaxed);
    case KKT_OPTION_VALIDATE_CU_SEQLENS: return g_validate_cu_seqlens.load(std::memory_order_relaxed);
    }
    return -1;
}

extern "C" const char* kkt_last_error(void) { return g_last_error.c_str(); }

extern "C" int kkt_version(void) { return KKT_VERSION_NUMBER; }
