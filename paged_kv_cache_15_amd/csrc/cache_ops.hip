// Cache writes into the paged pool: reshape_and_cache and copy-on-write block copies.
//
// deepsonar "PagedAttention de vLLM …" §2.2: each new token's K/V lands in its
// sequence's current block at the next free offset; §2.3: a shared block is copied
// before it is written.  deeplearn.tn "PagedAttention : comment optimiser la mémoire
// GPU …", worked example: the token written after a full block goes to offset 0 of
// a freshly taken block anywhere in the pool.
//
// Pool layout (chunk X = 16 bytes / element size, BS = block size 1, 16 or 32; a block of
// 32 tokens is two 16-token sub-blocks one after the other, TB = min(BS, 16) tokens each):
//   K [block][kv_head][BS / TB][head_dim / X][TB][X]   V [block][kv_head][BS / TB][head_dim][TB]

#include <hip/hip_runtime.h>

#include "common.h"

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

// One thread per (token, KV head, 16-byte chunk of head_dim).  The key chunk is one
// 16-byte store; the value chunk scatters its X elements down X rows of the
// transposed V tile (stride TB elements; one 16-byte store when BS is 1).
template <typename T, int BS>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const T* __restrict__ key, const T* __restrict__ value, int64_t key_stride,
    int64_t value_stride, T* __restrict__ k_pool, T* __restrict__ v_pool,
    const int32_t* __restrict__ slot_mapping, int32_t num_tokens, int32_t kv_heads,
    int32_t head_dim, int64_t num_slots) {
    constexpr int X = 16 / sizeof(T);
    const int chunks = head_dim / X;
    const int64_t per_token = (int64_t)kv_heads * chunks;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)num_tokens * per_token) return;
    const int32_t t = (int32_t)(idx / per_token);
    const int32_t r = (int32_t)(idx - (int64_t)t * per_token);
    const int32_t h = r / chunks, c = r - h * chunks;
    // the token's chunks do not depend on its slot: all three loads are in flight together
    const int32_t slot = slot_mapping[t];
    const i32x4 kc = *reinterpret_cast<const i32x4*>(key + t * key_stride + (int64_t)h * head_dim + c * X);
    const i32x4 vc = *reinterpret_cast<const i32x4*>(value + t * value_stride + (int64_t)h * head_dim + c * X);
    // (an empty use keeps the compiler from sinking the two loads below the slot test)
    asm volatile("" ::"v"(kc), "v"(vc));
    if (slot < 0 || (int64_t)slot >= num_slots) return;
    constexpr int TB = BS < 16 ? BS : 16;   // tokens per sub-block
    const int64_t blk = slot / BS;
    const int32_t sub = (slot % BS) / TB, off = slot % TB;

    const int64_t region = (blk * kv_heads + h) * (BS / TB) + sub;   // (block, head, sub-block)
    T* kdst = k_pool + ((region * chunks + c) * TB + off) * X;
    *reinterpret_cast<i32x4*>(kdst) = kc;

    T* vdst = v_pool + (region * head_dim + (int64_t)c * X) * TB + off;
    if constexpr (BS == 1) {
        *reinterpret_cast<i32x4*>(vdst) = vc;
    } else {
        T ve[X];
        __builtin_memcpy(ve, &vc, 16);
#pragma unroll
        for (int e = 0; e < X; ++e) vdst[e * TB] = ve[e];
    }
}

// One workgroup per (pair, K or V): copies a whole block (all heads, all slots).
__global__ __launch_bounds__(256) void copy_blocks_kernel(char* __restrict__ k_pool,
                                                          char* __restrict__ v_pool,
                                                          const int32_t* __restrict__ pairs,
                                                          int32_t num_blocks, int64_t block_bytes) {
    const int32_t src = pairs[2 * blockIdx.x], dst = pairs[2 * blockIdx.x + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
    char* base = blockIdx.y == 0 ? k_pool : v_pool;
    const i32x4* s = reinterpret_cast<const i32x4*>(base + src * block_bytes);
    i32x4* d = reinterpret_cast<i32x4*>(base + dst * block_bytes);
    const int64_t n = block_bytes / 16;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) d[i] = s[i];
}

template <typename T>
void launch_reshape(const paged_kv_pool_desc* desc, const void* key, const void* value,
                    int64_t key_stride, int64_t value_stride, void* k_pool, void* v_pool,
                    const int32_t* slot_mapping, int32_t num_tokens, int64_t num_slots,
                    int64_t grid, hipStream_t st) {
    const T* k = static_cast<const T*>(key);
    const T* v = static_cast<const T*>(value);
    T* kp = static_cast<T*>(k_pool);
    T* vp = static_cast<T*>(v_pool);
    const dim3 g((unsigned)grid), b(256);
    switch (desc->block_size) {
        case 1:
            reshape_and_cache_kernel<T, 1><<<g, b, 0, st>>>(k, v, key_stride, value_stride, kp, vp,
                slot_mapping, num_tokens, desc->num_kv_heads, desc->head_dim, num_slots);
            break;
        case 32:
            reshape_and_cache_kernel<T, 32><<<g, b, 0, st>>>(k, v, key_stride, value_stride, kp, vp,
                slot_mapping, num_tokens, desc->num_kv_heads, desc->head_dim, num_slots);
            break;
        default:
            reshape_and_cache_kernel<T, 16><<<g, b, 0, st>>>(k, v, key_stride, value_stride, kp, vp,
                slot_mapping, num_tokens, desc->num_kv_heads, desc->head_dim, num_slots);
            break;
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

paged_kv_status launch_status(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        pkv::set_error("%s launch failed: %s", what, hipGetErrorString(e));
        return PAGED_KV_ERR_HIP;
    }
    return PAGED_KV_OK;
}

}  // namespace

extern "C" {

paged_kv_status reshape_and_cache(const paged_kv_pool_desc* desc, const void* key,
                                  const void* value, int64_t key_stride, int64_t value_stride,
                                  void* k_pool, void* v_pool, const int32_t* slot_mapping,
                                  int32_t num_tokens, void* stream) {
    pkv::clear_error();
    if (!pkv::kernel_desc(desc, false)) return PAGED_KV_ERR_INVALID_ARG;
    if (num_tokens < 0) { pkv::set_error("num_tokens < 0"); return PAGED_KV_ERR_INVALID_ARG; }
    if (num_tokens == 0) return PAGED_KV_OK;
    if (!key || !value || !k_pool || !v_pool || !slot_mapping) {
        pkv::set_error("null pointer argument");
        return PAGED_KV_ERR_INVALID_ARG;
    }
    const int eb = pkv::elem_bytes(desc->dtype);
    const int64_t row = (int64_t)desc->num_kv_heads * desc->head_dim;
    if (key_stride < row || value_stride < row || (key_stride * eb) % 16 || (value_stride * eb) % 16) {
        pkv::set_error("token strides (%lld, %lld) must be >= heads*dim = %lld and 16-byte multiples",
                       (long long)key_stride, (long long)value_stride, (long long)row);
        return PAGED_KV_ERR_INVALID_ARG;
    }
    if (!aligned16(key) || !aligned16(value) || !aligned16(k_pool) || !aligned16(v_pool)) {
        pkv::set_error("key, value and pool pointers must be 16-byte aligned");
        return PAGED_KV_ERR_INVALID_ARG;
    }
    const int64_t threads = (int64_t)num_tokens * desc->num_kv_heads * (desc->head_dim * eb / 16);
    const int64_t grid = (threads + 255) / 256;
    if (grid > INT32_MAX) { pkv::set_error("too many tokens for one launch"); return PAGED_KV_ERR_UNSUPPORTED; }
    const int64_t num_slots = (int64_t)desc->num_blocks * desc->block_size;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (eb == 4) launch_reshape<uint32_t>(desc, key, value, key_stride, value_stride, k_pool, v_pool,
                                          slot_mapping, num_tokens, num_slots, grid, st);
    else launch_reshape<uint16_t>(desc, key, value, key_stride, value_stride, k_pool, v_pool,
                                  slot_mapping, num_tokens, num_slots, grid, st);
    return launch_status("reshape_and_cache");
}

paged_kv_status paged_kv_copy_blocks(const paged_kv_pool_desc* desc, void* k_pool, void* v_pool,
                                     const int32_t* pairs, int32_t n, void* stream) {
    pkv::clear_error();
    if (!pkv::valid_desc(desc)) return PAGED_KV_ERR_INVALID_ARG;
    if (n < 0) { pkv::set_error("n < 0"); return PAGED_KV_ERR_INVALID_ARG; }
    if (n == 0) return PAGED_KV_OK;
    if (!k_pool || !v_pool || !pairs) { pkv::set_error("null pointer argument"); return PAGED_KV_ERR_INVALID_ARG; }
    if (!aligned16(k_pool) || !aligned16(v_pool)) {
        pkv::set_error("pool pointers must be 16-byte aligned");
        return PAGED_KV_ERR_INVALID_ARG;
    }
    const int64_t block_bytes = (int64_t)desc->num_kv_heads * desc->block_size * desc->head_dim *
                                pkv::elem_bytes(desc->dtype);
    copy_blocks_kernel<<<dim3((unsigned)n, 2), dim3(256), 0, reinterpret_cast<hipStream_t>(stream)>>>(
        (char*)k_pool, (char*)v_pool, pairs, desc->num_blocks, block_bytes);
    return launch_status("copy_blocks");
}

}  // extern "C"
