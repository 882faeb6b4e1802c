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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16 with round-to-nearest-even: gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// Exact-form GeLU, v * Phi(v), Phi the standard normal CDF (列并行 tutorial,
// MLP 应用), evaluated in fp32 as
//   Phi(-|v|) = erfc(x) / 2,  x = |v| / sqrt(2),
//   erfc(x) ~= t (a1 + a2 t + a3 t^2 + a4 t^3 + a5 t^4) exp(-x^2),  t = 1 / (1 + p x),
// the rational-exponential approximation of Abramowitz & Stegun, Handbook of
// Mathematical Functions, formula 7.1.26 (after Hastings), whose absolute
// error in erf/erfc is at most 1.5e-7 for x >= 0.  The argument is carried
// as z = |v| sqrt(log2(e) / 2), so that exp(-x^2) = exp(-v^2 / 2) = 2^(-z^2)
// is one multiply and one v_exp_f32, and p / sqrt(log2 e) and a_i / 2 are
// folded constants.  Phi(v) = 1 - Phi(-|v|) for v >= 0, so
//   GeLU(v) = max(v, 0) - |v| Phi(-|v|)
// (one max and one fma; |v| is clamped to the largest float so that
// GeLU(+inf) = +inf and GeLU(-inf) = 0; a NaN stays NaN through the tail).  The tail term is computed
// directly: no cancellation for v << 0.  Max |GeLU error| over fp32 inputs
// 3.3e-7 in a float32 emulation (the same class as v/2 (1 + erff(v/sqrt2)) in
// fp32) at about a quarter of that form's instruction count.
struct NormalTail {
  float tail;  // Phi(-|v|)
  float e;     // exp(-v^2 / 2)
};
__device__ __forceinline__ NormalTail normal_tail(float v) {
  const float z = __builtin_fabsf(v) * 0.84932180028801904f;         // sqrt(log2(e) / 2)
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.27273748087922250f, z, 1.0f));  // p / sqrt(log2 e)
  float p = __builtin_fmaf(t, 0.5307027145f, -0.7265760135f);          // a5 / 2, a4 / 2
  p = __builtin_fmaf(t, p, 0.7107068705f);                             // a3 / 2
  p = __builtin_fmaf(t, p, -0.142248368f);                             // a2 / 2
  p = __builtin_fmaf(t, p, 0.127414796f);                              // a1 / 2
  const float e = __builtin_amdgcn_exp2f(-(z * z));
  return {(p * t) * e, e};
}

__device__ __forceinline__ float gelu_f32(float v) {
  const float tail = normal_tail(v).tail;
  // max(v, 0) as a signed-integer max of the bits (a negative float is a
  // negative integer): one instruction, where fmaxf also quiets NaN inputs
  const float pos = __builtin_bit_cast(float, max(__builtin_bit_cast(int, v), 0));
  return __builtin_fmaf(-__builtin_fminf(__builtin_fabsf(v), 3.402823466e38f), tail, pos);
}

// d/dv GeLU(v) = Phi(v) + v phi(v), phi(v) = exp(-v^2/2) / sqrt(2 pi) the
// standard normal density (the product rule on v Phi(v)); Phi as above, the
// density from the same exponential.
__device__ __forceinline__ float gelu_grad_f32(float v) {
  const NormalTail n = normal_tail(v);
  const float cdf = v >= 0.0f ? 1.0f - n.tail : n.tail;
  return __builtin_fmaf(v * 0.39894228040143268f, n.e, cdf);
}

// SiLU(z) = z * sigma(z) = z / (1 + exp(-z)), sigma the logistic function
// (the gate of the SwiGLU variant): one v_exp_f32 and one v_rcp_f32.  For
// z << 0 the exponential overflows to +inf and the reciprocal gives 0.
__device__ __forceinline__ float silu_f32(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
}

// ---- global->LDS copies and explicit LDS synchronisation (gfx950) --------

// Workgroup barrier with no memory fence: the compiler may not move memory
// operations across it, and inserts no waits for it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// One 1 KiB global->LDS copy: lane t's 16 bytes from `src` land at LDS byte
// address lds_addr + 16 t (lds_addr uniform, in M0).  Issued as inline
// assembly so that the compiler does not treat it as an LDS store: left to
// itself it would make later LDS reads of *other* stages wait for every copy
// in flight (s_waitcnt vmcnt(0)), which defeats the pipeline.  Ordering
// against LDS reads is explicit instead: wait_vmcnt + lds_barrier.  The LDS
// address is an input bound to M0 ("{m0}"), so the compiler writes M0 itself
// and knows the instruction reads it; the s_nop separates that write from
// the copy.
__device__ __forceinline__ void copy_to_lds(const void* src, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds_addr));
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const void*)(p)));
}

// s_waitcnt vmcnt(N) only (expcnt and lgkmcnt fields at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

}  // namespace tpk
