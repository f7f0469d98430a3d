// Device-side types and small helpers shared by the fldce kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fldce {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
// Largest sum over one 128-wide vocabulary slab of exp(z - r), r = the row's
// target logit, for which a row's backward operand stays relative to r: 2^43.
// Below it every such exponential is at most 2^43 (z - r <= 29.8 nats), and
// a row's sum of up to 2^24 slabs stays far inside float32; a row with a
// larger slab sum (some logit 25-30 nats or more above the target logit) is
// redone relative to its logsumexp.
constexpr float kRefSumMax = 8796093022208.0f;
constexpr float kLn2 = 0.6931471805599453f;

// Global / LDS address-space casts for the direct global->LDS load builtin.
#define FLDCE_GPTR(p) ((const void __attribute__((address_space(1)))*)(p))
#define FLDCE_LPTR(p) ((void __attribute__((address_space(3)))*)(p))

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wave-wide (64 lanes) reductions through cross-lane shuffles.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Combine two (max, sum-exp) pairs: result max M and sum relative to M.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) { m = M; s = 0.f; return; }
  s = s * fast_exp2((m - M) * kLog2e) + s2 * fast_exp2((m2 - M) * kLog2e);
  m = M;
}

__host__ __device__ constexpr int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ constexpr int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// Split count for a split-K GEMM with `tiles` output tiles and k_tiles K
// tiles, at most max_splits: 1 when the tiles fill the 256 CUs at least
// once; else minimises the waves of work per split (ceil(tiles * S / 256) /
// S, plus a small charge per split for the fp32 partials), keeping >= 8 K
// tiles per split.  Used by the host to size
// the grid and the partial buffer, and by the kernels on the device once the
// number of active tiles is known.
__host__ __device__ inline int choose_splits(int64_t tiles, int64_t k_tiles, int max_splits) {
  // With a full wave of tiles already, a partly filled last wave costs little
  // (measured: its CUs run at a higher clock and with less memory contention),
  // so more splits would only add partial-sum traffic.
  if (tiles >= 256) return 1;
  int best = 1;
  double bestc = 1e300;
  for (int S = 1; S <= max_splits; ++S) {
    if (k_tiles / S < 8) break;
    const double waves = (double)((tiles * S + 255) / 256);
    const double c = waves / S + 0.02 * S;
    if (c < bestc - 1e-12) {
      bestc = c;
      best = S;
    }
  }
  return best;
}

}  // namespace fldce
