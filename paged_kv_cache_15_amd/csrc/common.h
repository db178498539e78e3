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

// Extra conditions the device kernels need (block size 1, 16 or 32; for attention,
// head_dim 64, 128 or 256).
bool kernel_desc(const paged_kv_pool_desc* d, bool attention);

constexpr int kTileTokens = 16;   // attention works on 16-token tiles of a sequence

// Resident waves per SIMD of the attention kernels for head_dim d, element bytes e.
// Stream-K kernels: 1 above head_dim 64 (measured: fewer, longer slices stream faster
// once a wave's two tiles in flight are 8 KiB or more); the MFMA one at head_dim 64 2,
// with three 4 KiB tiles in flight (1.5% faster than 3 waves with two, in three
// alternating same-machine runs); else as their fixed-partition twins.  Fixed-partition
// kernels, by their registers: MFMA 3 up to head_dim 128 and 1 at 256; VALU (registers
// grow with the 16-byte loads per lane of a tile, ni) 3 up to 4 loads, 2 up to 8 and 1
// beyond.
constexpr int kernel_waves_per_simd(int d, int e, bool mfma, bool streamk) {
    return streamk && d > 64            ? 1
           : streamk && mfma && d == 64 ? 2
           : mfma                       ? (d > 128 ? 1 : 3)
                                        : (d * e / 64 <= 4 ? 3 : d * e / 64 <= 8 ? 2 : 1);
}
constexpr int kDefaultPartitionTokens = 512;

// What the launch plans need to know about the device they launch on.
struct DeviceShape {
    int compute_units;   // hipDeviceAttributeMultiprocessorCount
    int xcds;            // accelerator dies the compute units are spread over (workgroup b
                         // runs on die b % xcds); compute_units / 32 on gfx950, else 1
    bool mi355x_spx;     // gfx950 with all 256 compute units in one device: the shape the
                         // stream-K XCD slice weights were measured on
};
// The current device's shape (cached per device).  With no usable device it returns
// default_device_shape(), the MI355X in SPX mode, so that host-only sizing calls still
// answer; no kernel can be launched then anyway.
DeviceShape device_shape();
DeviceShape default_device_shape();

}  // namespace pkv
