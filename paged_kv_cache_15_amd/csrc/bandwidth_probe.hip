// Streaming-read probe: the measured HBM read bandwidth that the decode kernels' roofline
// is also stated against (next to the 8 TB/s of the part's specification).
//
// The loads are those of the attention kernels' K/V stream: 16 bytes per lane, each
// wave instruction reading 1 KiB contiguous, nontemporal, 16 instructions in flight per
// wave, two waves per SIMD of the device, each wave streaming its own contiguous run.  The XOR of everything read is stored only if it equals a value no probe
// buffer produces in practice, which keeps the loads without writing anything.

#include <hip/hip_runtime.h>

#include "common.h"

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

constexpr int kUnroll = 16;   // 1 KiB wave loads in flight per wave

// Wave w of W reads the contiguous chunks [C w / W, C (w + 1) / W) of the C 1 KiB chunks
// of the buffer (each wave streams its own run, as a decode wave streams its slice of
// tiles); the last partial chunk, if any, is read by wave 0.
__global__ __launch_bounds__(256) void stream_read_kernel(const i32x4* __restrict__ buf, int64_t n16,
                                                          int32_t* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int64_t waves = (int64_t)gridDim.x * 4;
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t chunks = n16 / 64;
    const int64_t c1 = chunks * (w + 1) / waves;
    int64_t c = chunks * w / waves;
    i32x4 acc = {0, 0, 0, 0};
    for (; c + kUnroll <= c1; c += kUnroll) {
        i32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + (c + u) * 64 + lane);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
    for (; c < c1; ++c) acc ^= __builtin_nontemporal_load(buf + c * 64 + lane);
    if (w == 0)
        for (int64_t i = chunks * 64 + lane; i < n16; i += 64) acc ^= buf[i];
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
    // two waves per SIMD (a block's four waves land one on each SIMD of a compute unit)
    const int blocks = pkv::device_shape().compute_units * 2;
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
