// Streaming-read probe: the measured HBM read bandwidth that the decode kernels' roofline
// is also stated against (next to the 8 TB/s of the part's specification).
//
// The loads are those of the attention kernels' K/V stream: 16 bytes per lane, each
// wave instruction reading 1 KiB contiguous, nontemporal, several instructions in
// flight per wave, one wave per SIMD slot of the device and a grid-stride walk over the
// buffer.  The XOR of everything read is stored only if it equals a value no probe
// buffer produces in practice, which keeps the loads without writing anything.

#include <hip/hip_runtime.h>

#include "common.h"

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

constexpr int kUnroll = 8;   // 16-byte loads in flight per lane

__global__ __launch_bounds__(256) void stream_read_kernel(const i32x4* __restrict__ buf, int64_t n16,
                                                          int32_t* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    i32x4 acc = {0, 0, 0, 0};
    for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
        i32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(buf + i);
    const int x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (x == 0x5eed1e55) sink[0] = x;
}

}  // namespace

extern "C" {

paged_kv_status paged_kv_read_bandwidth_probe(const void* buf, size_t bytes, void* sink,
                                              void* stream) {
    pkv::clear_error();
    if (!buf || !sink || bytes == 0 || bytes % 16 || reinterpret_cast<uintptr_t>(buf) % 16 ||
        reinterpret_cast<uintptr_t>(sink) % 4) {
        pkv::set_error("need a 16-byte aligned buffer of a positive multiple of 16 bytes and a sink");
        return PAGED_KV_ERR_INVALID_ARG;
    }
    const int blocks = pkv::device_shape().compute_units * 4;   // 4 waves per block: one per SIMD
    stream_read_kernel<<<dim3(blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream)>>>(
        static_cast<const i32x4*>(buf), (int64_t)(bytes / 16), static_cast<int32_t*>(sink));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        pkv::set_error("stream read probe launch failed: %s", hipGetErrorString(e));
        return PAGED_KV_ERR_HIP;
    }
    return PAGED_KV_OK;
}

}  // extern "C"
