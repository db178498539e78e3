// SHA-256 (FIPS 180-4, "Secure Hash Standard", §4.1.2 functions, §4.2.2 constants,
// §5.1.1 padding, §6.2.2 hash computation), for the chained block hashes of the
// prefix cache.  Incremental: update() any number of times, then final().
#pragma once

#include <cstddef>
#include <cstdint>

namespace pkv {

class Sha256 {
public:
    Sha256();
    void update(const void* data, size_t n);
    void final(uint8_t out[32]);

private:
    void block(const uint8_t* p);
    uint32_t h_[8];
    uint8_t buf_[64];
    size_t fill_ = 0;
    uint64_t bits_ = 0;
};

}  // namespace pkv
