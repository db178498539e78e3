// Internal helpers shared by the library's translation units (host side).
#pragma once

#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <string>

#include "paged_kv.h"

namespace pkv {

// Thread-local detail of the last failure, returned by paged_kv_last_error().
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();

inline int elem_bytes(int32_t dtype) {
    switch (dtype) {
        case PAGED_KV_F32: return 4;
        case PAGED_KV_F16: return 2;
        case PAGED_KV_BF16: return 2;
        default: return 0;
    }
}

// Checks every field of a descriptor; on failure records why and returns false.
bool valid_desc(const paged_kv_pool_desc* d);

// Extra conditions the device kernels need (block size 16, supported head dims).
bool kernel_desc(const paged_kv_pool_desc* d, bool attention);

constexpr int kKernelBlockSize = 16;
constexpr int kDefaultPartitionTokens = 512;

}  // namespace pkv
