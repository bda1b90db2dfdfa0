// Host set-up values (setup.cpp).
#pragma once
#include <stdint.h>

#include <vector>

namespace jolt {

uint64_t splitmix_word(uint64_t key, uint64_t n);
uint64_t stream_key(uint64_t seed, uint64_t stream);
void gaussians(uint64_t seed, uint64_t stream, uint64_t start, uint64_t count, double *out);
// D x D rotation, row-major, cached per (D, seed)
const std::vector<double> &rotation(int D, uint64_t seed);
// eps^2(b) for b = 0..8 (eps^2(0) = 1), cached per D
const std::vector<double> &eps2_table(int D);

}  // namespace jolt
