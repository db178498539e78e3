// Device-side helpers shared by the decode attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "common.h"

namespace pkv_dev {

typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4;

constexpr int kTile = 16;                   // tokens per tile: the 16 rows of one MFMA block
constexpr int kWaves = 4;                   // waves per partition workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -INFINITY;
constexpr float kRescaleSlack = 8.f;        // log2 units: weights stay below 2^8

enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-bit storage bits -> float
template <int DT>
__device__ __forceinline__ float bits_to_f32(uint32_t b) {
    if constexpr (DT == DT_BF16) return __uint_as_float(b << 16);
    else if constexpr (DT == DT_F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
    else return __uint_as_float(b);
}

// float -> 16-bit storage bits, round to nearest even
template <int DT>
__device__ __forceinline__ uint16_t f32_to_bits16(float f) {
    if constexpr (DT == DT_BF16) return __builtin_bit_cast(uint16_t, (__bf16)f);
    else return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Partial results that another workgroup of the same launch merges may cross XCDs,
// whose L2 caches are not kept coherent with each other inside a kernel.  They are
// written and read with agent-scope relaxed atomics, which the compiler emits as
// write-through stores and coherent loads (sc1); publishing them then only needs the
// stores to have completed before a counter is bumped.  (An agent-scope release fence
// would instead write back the XCD's whole L2, and such write-backs serialise across
// the thousands of partial results of one launch.)
__device__ __forceinline__ void put_coherent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float get_coherent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Every vector memory operation this wave issued has completed (vmcnt counts stores
// too on this architecture); the clobber keeps the compiler from moving memory
// operations across it.
__device__ __forceinline__ void wait_memory_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int OUT_DT>
__device__ __forceinline__ void store_out(void* out, int64_t i, float v) {
    if constexpr (OUT_DT == DT_F32) static_cast<float*>(out)[i] = v;
    else static_cast<uint16_t*>(out)[i] = f32_to_bits16<OUT_DT>(v);
}

// max over the lanes that share lane % 16 (xor 16, 32)
__device__ __forceinline__ float max_across_quads(float v) {
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}
__device__ __forceinline__ float sum_across_quads(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

// Read-only int32 through the scalar data cache: block tables and context lengths are
// never written while a kernel runs, and a scalar load keeps the per-tile lookups off the
// vector memory counter, so waiting for one never waits for the K/V loads in flight.
__device__ __forceinline__ int32_t sload(const int32_t* p, int64_t i) {
    return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

// Waves per SIMD the attention kernels are compiled for (a wave's registers must fit in
// 512 / waves): two tiles of K/V in flight plus the accumulators and the query.  The
// host plans stream-K launches with the same numbers (pkv::kernel_waves_per_simd).
template <int D, bool STREAMK>
constexpr int mfma_waves_per_simd() { return pkv::kernel_waves_per_simd(D, 2, true, STREAMK); }
template <int D, int E, bool STREAMK>
constexpr int valu_waves_per_simd() { return pkv::kernel_waves_per_simd(D, E, false, STREAMK); }

// Tiles in flight per wave in the stream-K MFMA kernel (ring of load buffers).  Two:
// rings of 3 and 4 measured no faster at one wave per SIMD (the tiles in flight per CU
// are not what limits the stream).  Three at head_dim 64 (4 KiB tiles, two waves per
// SIMD).
template <int D>
constexpr int stream_depth() { return D == 64 ? 3 : 2; }

// Block size 1: every token of a tile sits in its own block.  Lane l gets the block of
// token 16*it + (l & 15) of the table row (ids read through the scalar cache; tokens at
// or past ctx, which must be >= 1, take the id of token ctx - 1).  An id outside
// [0, num_blocks) sets `bad` and reads block 0.
__device__ __forceinline__ int32_t lane_block_bs1(const int32_t* row, int it, int ctx,
                                                  int num_blocks, int lane, bool& bad) {
    int32_t ids[kTile];
#pragma unroll
    for (int j = 0; j < kTile; ++j) ids[j] = sload(row, min(kTile * it + j, ctx - 1));
    bool any = false;
#pragma unroll
    for (int j = 0; j < kTile; ++j) any |= (uint32_t)ids[j] >= (uint32_t)num_blocks;
    bad = any;
    const int tok = lane & (kTile - 1);
    int32_t id = ids[0];
#pragma unroll
    for (int j = 1; j < kTile; ++j) id = tok == j ? ids[j] : id;
    return (uint32_t)id < (uint32_t)num_blocks ? id : 0;
}

// Block size 1 stores V token-major (a block's [head_dim][1] is one token's row), while
// the value products want each lane to hold several tokens of one dim.  A wave passes its
// tile through its own LDS rows of `ldw` elements: lane l wrote 16-byte chunks
// 4*i + l/16 of token l & 15 (the K-style load), then reads single elements back.
// LDS operations of one wave complete in order, so no barrier is needed; rows are padded
// by 16 bytes so that the element reads of one instruction hit distinct banks.
template <typename T, int NCH>
__device__ __forceinline__ void lds_put_rows(T* rows, int ldw, int lane, const i32x4 (&raw)[NCH]) {
    constexpr int X = 16 / sizeof(T);
#pragma unroll
    for (int i = 0; i < NCH; ++i)
        *reinterpret_cast<i32x4*>(rows + (lane & 15) * ldw + (4 * i + (lane >> 4)) * X) = raw[i];
}

// Block size 1, whole-row loads.  A token's K (or V) row for one head is D contiguous
// elements, D / 8 chunks of 16 bytes.  Load i of lane l reads chunk l % (D / 8) of the
// tile's token (512 / D) i + l / (D / 8), so every load instruction reads whole rows (a
// 256-byte row per 16 lanes at head_dim 128).  Loads in the score product's own operand
// layout (16 tokens per instruction, 64 bytes of each) streamed at 0.56 of the HBM peak
// on the GQA workload, whole rows at 0.71.  The rows then pass through the wave's LDS.
// Block of the lane's token in load i, from idv = lane_block_bs1(...) (lane j < 16 holds
// the block of the tile's token j).
template <int D>
__device__ __forceinline__ int32_t load_id_bs1(int32_t idv, int i, int lane) {
    return __shfl(idv, (512 / D) * i + lane / (D / 8));
}
// Lane l's chunk of load i into the wave's LDS rows ([token][element], rows of ldw).
template <int D, int NL>
__device__ __forceinline__ void lds_put_whole_rows(uint16_t* rows, int ldw, int lane,
                                                   const i32x4 (&raw)[NL]) {
    constexpr int RPI = 512 / D, CPR = D / 8;
#pragma unroll
    for (int i = 0; i < NL; ++i)
        *reinterpret_cast<i32x4*>(rows + (RPI * i + lane / CPR) * ldw + (lane % CPR) * 8) = raw[i];
}

}  // namespace pkv_dev
