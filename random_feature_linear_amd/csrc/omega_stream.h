// The random projection's Gaussian stream, shared by the host generator
// (dark_prf_omega) and the device generator (dark_prf_omega_device): SplitMix64
// (Steele, Lea and Flood 2014) over the counter i + 1, the top 53 bits as a
// uniform in (0, 1], and Box-Muller pairs (k even: cosine, k odd: sine).  The
// package README's section "Kernel" draws each omega_j from a standard
// Gaussian; section "Projection lifecycle" makes a projection reproducible from
// a seed.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace dk {

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}
__host__ __device__ inline double uniform_at(uint64_t seed, uint64_t i) {
  const uint64_t x = mix64(seed + (i + 1) * 0x9E3779B97F4A7C15ULL);
  return ((double)(x >> 11) + 1.0) * 0x1.0p-53;
}
__host__ __device__ inline double normal_at(uint64_t seed, uint64_t k) {
  const uint64_t p = k >> 1;
  const double u1 = uniform_at(seed, 2 * p);
  const double u2 = uniform_at(seed, 2 * p + 1);
  const double rad = sqrt(-2.0 * log(u1));
  const double ang = 2.0 * 3.14159265358979323846 * u2;
  return (k & 1) ? rad * sin(ang) : rad * cos(ang);
}

}  // namespace dk
