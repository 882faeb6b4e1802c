// Device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace tpk {

// Calls f(std::integral_constant<int, I>{}) for I = 0 .. N-1, fully unrolled in
// the front end, so that arrays indexed by I are register-promoted before any
// loop pass runs.
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  [&]<int... I>(std::integer_sequence<int, I...>) __attribute__((always_inline)) {
    (f(std::integral_constant<int, I>{}), ...);
  }(std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// Exact GeLU, v * Phi(v) = v/2 * (1 + erf(v / sqrt 2)), with the device erff.
__device__ __forceinline__ float gelu_f32(float v) {
  return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f));
}

}  // namespace tpk
