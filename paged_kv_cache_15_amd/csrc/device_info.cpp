// Shape of the current HIP device, as the attention launch plans need it.
//
// Read once per device (compute-unit count from hipDeviceGetAttribute, the ISA name from
// hipGetDeviceProperties) and cached: the plans run on every launch.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "common.h"

namespace pkv {

namespace {

constexpr int kMaxDevices = 64;
constexpr int kCusPerXcdGfx950 = 32;   // compute units per accelerator die on gfx950
constexpr int kMi355xCus = 256;        // all eight dies in one device (SPX partition mode)

// packed: compute units (bits 0-15), dies (16-23), MI355X SPX flag (bit 24); 0 = not read
std::atomic<int64_t> g_shape[kMaxDevices];

int64_t pack(const DeviceShape& s) {
    return (int64_t)s.compute_units | (int64_t)s.xcds << 16 | (int64_t)(s.mi355x_spx ? 1 : 0) << 24;
}

DeviceShape unpack(int64_t v) {
    return DeviceShape{(int)(v & 0xFFFF), (int)((v >> 16) & 0xFF), ((v >> 24) & 1) != 0};
}

DeviceShape read_shape(int dev) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return default_device_shape();
    hipDeviceProp_t prop;
    bool gfx950 = false;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess)
        gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    DeviceShape s;
    s.compute_units = cus;
    s.xcds = gfx950 && cus % kCusPerXcdGfx950 == 0 ? cus / kCusPerXcdGfx950 : 1;
    if (s.xcds > 8) s.xcds = 8;
    s.mi355x_spx = gfx950 && cus == kMi355xCus;
    return s;
}

}  // namespace

DeviceShape default_device_shape() { return DeviceShape{kMi355xCus, 8, true}; }

DeviceShape device_shape() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();   // leave no sticky error for the caller's next HIP call
        return default_device_shape();
    }
    if (dev >= kMaxDevices) return read_shape(dev);
    int64_t v = g_shape[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        v = pack(read_shape(dev));
        g_shape[dev].store(v, std::memory_order_relaxed);
    }
    return unpack(v);
}

}  // namespace pkv
