// Memory-traffic reference for the fused chunk-local KKT + solve (64-token
// chunks, sequences of whole chunks).  It moves exactly the bytes one fused
// step moves, in the fused kernel's pattern, and does no arithmetic:
//   - one 64-row tile (one chunk of one head) per wave, four waves (four
//     heads of a chunk) per workgroup, in the fused kernel's XCD order: grids
//     of up to 1024 workgroups spread in contiguous ranges over the 8 XCDs,
//     larger ones keep all the workgroups of a chunk on one XCD with the
//     chunks round-robin over the XCDs (the heads of a token share the cache
//     lines of g and beta, so each line is fetched by one L2).  (The fused
//     kernel runs grids of up to 1024 tiles in one-wave workgroups; for this
//     kernel that form is slower, 7.3 vs 6.7 us at (1,8192,8,128), so the
//     reference keeps four waves);
//   - g and beta of the tile's rows first (one row per lane), then every key
//     row in 16-byte loads, all issued before any store;
//   - the tile's output rows written in whole-row 16-byte pieces with
//     non-temporal stores.
// Its time is a floor for any kernel with this data movement and this
// load-before-store dependency inside a wave on this machine; it is not part
// of the operation (bench.py times it as --op floor).
//
// Output: 16-byte piece c of output row (b, t, h) is piece c mod (key row
// bytes / 16) of key row (b, t, h), so that a test can check every byte.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kkt_floor.h"

namespace {

constexpr int kWave = 64;
constexpr int kRows = 64;        // rows of one tile
constexpr int kWavesPerGroup = 4;
constexpr uint32_t kContiguousMaxGroups = 1024;  // grids of up to this many workgroups: contiguous XCD ranges
constexpr int kNonTemporal = 2;  // cache-policy bit "nt", as on the fused kernel's output stores

using u32x4 = uint32_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    // raw (untyped) buffer, stride 0: accesses at or past `bytes` read 0 / are dropped
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

struct FloorArgs {
    const char* k;
    const float* g;
    const float* beta;
    char* out;
    int32_t H;
    int32_t chunks_per_row;
    uint32_t n_tiles;
    int64_t T;
    uint32_t n_groups;         // workgroups of the grid
    int32_t contiguous;        // 1: each XCD takes one contiguous range of workgroups' tiles
    int32_t log2_run;          // otherwise: runs of 2^log2_run workgroups stay on one XCD
    uint32_t remap_groups;     // workgroups in whole rounds of runs (the rest keep their order)
};

// Workgroup w runs on XCD w % 8 (the hardware's round-robin); the tile group
// it takes, as described at the top.
__device__ __forceinline__ uint32_t tile_group(const FloorArgs& a)
{
    const uint32_t w = blockIdx.x, xcd = w % 8, slot = w / 8;
    if (a.contiguous) {
        const uint32_t per = a.n_groups / 8, extra = a.n_groups % 8;
        return (xcd < extra) ? xcd * (per + 1) + slot : extra * (per + 1) + (xcd - extra) * per + slot;
    }
    if (w >= a.remap_groups) return w;
    const uint32_t lg = (uint32_t)a.log2_run;
    return ((((slot >> lg) << 3) + xcd) << lg) | (slot & ((1u << lg) - 1u));
}

// KRB: key row bytes (128, 256 or 512); ORB: output row bytes (128 or 256).
// The arguments are scalars, preloaded into SGPRs at wave launch (the
// library is built with -amdgpu-kernarg-preload-count=9), as the fused
// kernels' are: no kernel-argument load precedes a tile's first loads.
// p_bits: contiguous (bit 0), log2_run (bits 1-5); n_groups and
// remap_groups follow from the others.
template <int KRB, int ORB, int WAVES>
__global__ __launch_bounds__(kWave * WAVES) void stream_floor_kernel(const char* p_k, const float* p_g,
                                                                     const float* p_beta, char* p_out, uint32_t p_H,
                                                                     uint32_t p_cpr, uint32_t p_n_tiles, uint32_t p_T,
                                                                     uint32_t p_bits)
{
    FloorArgs a;
    a.k = p_k;
    a.g = p_g;
    a.beta = p_beta;
    a.out = p_out;
    a.H = (int32_t)p_H;
    a.chunks_per_row = (int32_t)p_cpr;
    a.n_tiles = p_n_tiles;
    a.T = (int64_t)p_T;
    a.n_groups = (p_n_tiles + WAVES - 1) / WAVES;
    a.contiguous = (int32_t)(p_bits & 1u);
    a.log2_run = (int32_t)((p_bits >> 1) & 31u);
    a.remap_groups = (a.n_groups >> (a.log2_run + 3)) << (a.log2_run + 3);
    constexpr int kPieces = KRB / 16;                   // 16-byte pieces of a key row
    constexpr int kPasses = kPieces > 16 ? kPieces / 16 : 1;
    constexpr int kOutPieces = ORB / 16;
    static_assert(kOutPieces <= 16, "one pass of 16 lanes per output row");
    const int lane = threadIdx.x % kWave;
    const uint32_t tile = tile_group(a) * WAVES + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (tile >= a.n_tiles) return;  // wave-uniform
    const uint32_t H = (uint32_t)a.H;
    const uint32_t chunk = tile / H;
    const uint32_t h = tile - chunk * H;
    const uint32_t b = chunk / (uint32_t)a.chunks_per_row;
    const uint32_t c = chunk - b * (uint32_t)a.chunks_per_row;
    const int64_t row0 = (int64_t)b * a.T + (int64_t)c * kRows;  // first token of the tile
    const int64_t first = row0 * H + h;                          // its (token, head) row index
    const uint32_t stride_k = H * KRB, stride_o = H * ORB, stride_s = H * 4u;

    // g and beta: one row per lane
    uint32_t gv = 0, bv = 0;
    if (a.g != nullptr) {
        gv = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.g + first, 63u * stride_s + 4u), lane * stride_s, 0, 0);
    }
    if (a.beta != nullptr) {
        bv = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.beta + first, 63u * stride_s + 4u), lane * stride_s, 0, 0);
    }

    // key rows: 16 lanes per row, 4 rows per instruction; lane piece cl (and
    // cl + 16 p); rows narrower than 16 pieces are read twice by the lane pairs
    // cl and cl + kPieces (the same lines, one fetch)
    const int gl = lane / 16, cl = lane % 16;
    const __amdgpu_buffer_rsrc_t k_rsrc = make_rsrc(a.k + first * KRB, 63u * stride_k + KRB);
    u32x4 v[16][kPasses];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t row = 4 * i + gl;
#pragma unroll
        for (int p = 0; p < kPasses; ++p) {
            const uint32_t piece = (kPieces >= 16) ? (uint32_t)(cl + 16 * p) : (uint32_t)(cl % kPieces);
            v[i][p] = __builtin_amdgcn_raw_buffer_load_b128(k_rsrc, row * stride_k + piece * 16, 0, 0);
        }
    }
    // g and beta, and the key pieces beyond the output row's width, are
    // read, not used: keep the loads
    asm volatile("" ::"v"(gv), "v"(bv));
#pragma unroll
    for (int i = 0; i < 16; ++i) {
#pragma unroll
        for (int p = 1; p < kPasses; ++p) asm volatile("" ::"v"(v[i][p]));
    }

    // output rows: lane cl writes piece cl (only the first kOutPieces lanes
    // of each row when the row is narrower than 16 pieces)
    const __amdgpu_buffer_rsrc_t o_rsrc = make_rsrc(a.out + first * ORB, 63u * stride_o + ORB);
    if (cl < kOutPieces) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t row = 4 * i + gl;
            __builtin_amdgcn_raw_buffer_store_b128(v[i][0], o_rsrc, row * stride_o + cl * 16, 0, kNonTemporal);
        }
    }
}

template <int KRB, int ORB>
hipError_t launch(FloorArgs a, hipStream_t stream)
{
    const uint32_t waves = kWavesPerGroup;
    a.n_groups = (a.n_tiles + waves - 1) / waves;
    a.contiguous = a.n_groups <= kContiguousMaxGroups ? 1 : 0;
    const uint32_t per_chunk = ((uint32_t)a.H + waves - 1) / waves;  // workgroups per chunk
    int lg = 0;
    while ((2u << lg) <= per_chunk && lg < 16) ++lg;
    a.log2_run = lg;
    a.remap_groups = (a.n_groups >> (lg + 3)) << (lg + 3);
    hipLaunchKernelGGL((stream_floor_kernel<KRB, ORB, kWavesPerGroup>), dim3(a.n_groups), dim3(kWave * kWavesPerGroup),
                       0, stream, a.k, a.g, a.beta, a.out, (uint32_t)a.H, (uint32_t)a.chunks_per_row, a.n_tiles,
                       (uint32_t)a.T, (uint32_t)a.contiguous | ((uint32_t)a.log2_run << 1));
    return hipGetLastError();
}

}  // namespace

extern "C" int kkt_floor_copy(const void* k, const float* g, const float* beta, int64_t B, int64_t T, int64_t H,
                              int64_t key_row_bytes, int64_t out_row_bytes, void* out, hipStream_t stream)
{
    if (k == nullptr || out == nullptr || B <= 0 || T <= 0 || H <= 0 || T % kRows != 0) return 1;
    if (key_row_bytes != 128 && key_row_bytes != 256 && key_row_bytes != 512) return 1;
    if (out_row_bytes != 128 && out_row_bytes != 256) return 1;
    // per-tile buffer ranges (64 rows of H heads) and tile indices fit in 32 bits
    if (kRows * H * key_row_bytes >= (1LL << 31) || kRows * H * out_row_bytes >= (1LL << 31) ||
        B * (T / kRows) * H >= (1LL << 31) || T >= (1LL << 31)) {
        return 1;
    }
    FloorArgs a;
    a.k = static_cast<const char*>(k);
    a.g = g;
    a.beta = beta;
    a.out = static_cast<char*>(out);
    a.H = (int32_t)H;
    a.chunks_per_row = (int32_t)(T / kRows);
    a.n_tiles = (uint32_t)(B * (T / kRows) * H);
    a.T = T;
    hipError_t e;
    if (key_row_bytes == 128) {
        e = out_row_bytes == 128 ? launch<128, 128>(a, stream) : launch<128, 256>(a, stream);
    } else if (key_row_bytes == 256) {
        e = out_row_bytes == 128 ? launch<256, 128>(a, stream) : launch<256, 256>(a, stream);
    } else {
        e = out_row_bytes == 128 ? launch<512, 128>(a, stream) : launch<512, 256>(a, stream);
    }
    return e == hipSuccess ? 0 : 2;
}
