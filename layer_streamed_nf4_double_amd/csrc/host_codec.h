// Host NF4 codec (nf4_host.cpp).
#pragma once
#include <stdint.h>

namespace lsn {
void nf4_levels(float out[16]);
// false if any input is NaN or infinite (nothing written then)
bool nf4_quantize(const float* w, uint64_t n, uint8_t* codes, float* absmax);
void nf4_dequantize_host(const uint8_t* codes, const float* absmax, uint64_t n, float* w);
}  // namespace lsn
