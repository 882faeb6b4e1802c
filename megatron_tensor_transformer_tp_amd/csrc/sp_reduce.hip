// Sequence-parallel boundary on one device (Megatron expert interview
// Level 2, M034): the SUM reduce-scatter half of the exchange.  Rank r's
// sequence shard of the summed row-parallel output, plus the per-token
// bias and residual of that shard:
//   out[m, n] = sum_{j < t} Z_j[r0 + m, n] + bias[n] + residual[m, n],  r0 = r * M / t.
//
// HBM-bound: algorithmic bytes = t * (M/t) * h * 4 (partials) + the bias and
// residual reads + (M/t) * h * out size.  Each thread owns 4 consecutive
// columns of one row (16-byte fp32 loads of every partial, summed in rank
// order, so the result is deterministic); consecutive threads take
// consecutive column groups, so every wave reads contiguous 1 KiB runs of
// each partial; grid-stride over the shard.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "kernels.h"

namespace tpk {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <typename T>
__device__ __forceinline__ void load4(const T* p, float (&v)[4]);
template <>
__device__ __forceinline__ void load4<float>(const float* p, float (&v)[4]) {
  const f32x4_t w = *reinterpret_cast<const f32x4_t*>(p);
  v[0] = w[0]; v[1] = w[1]; v[2] = w[2]; v[3] = w[3];
}
template <>
__device__ __forceinline__ void load4<uint16_t>(const uint16_t* p, float (&v)[4]) {
  const u32x2_t w = *reinterpret_cast<const u32x2_t*>(p);
  v[0] = __uint_as_float(w[0] << 16);
  v[1] = __uint_as_float(w[0] & 0xFFFF0000u);
  v[2] = __uint_as_float(w[1] << 16);
  v[3] = __uint_as_float(w[1] & 0xFFFF0000u);
}

__device__ __forceinline__ void store4(float* p, const float (&v)[4]) {
  *reinterpret_cast<f32x4_t*>(p) = f32x4_t{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ void store4(uint16_t* p, const float (&v)[4]) {
  *reinterpret_cast<u32x2_t*>(p) = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

template <typename IN, typename OUT, bool BIAS, bool RES>
__global__ __launch_bounds__(256) void sp_reduce_kernel(const SpPartials parts, int t, int64_t row0,
                                                        int64_t rows, int hidden,
                                                        const IN* __restrict__ bias,
                                                        const IN* __restrict__ residual,
                                                        OUT* __restrict__ out) {
  const int groups_per_row = hidden / 4;
  const int64_t total = rows * groups_per_row;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < total; i += 256ll * gridDim.x) {
    const int64_t m = i / groups_per_row;
    const int n = static_cast<int>(i - m * groups_per_row) * 4;
    const int64_t src = (row0 + m) * hidden + n;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j = 0; j < t; ++j) {
      float v[4];
      load4(parts.p[j] + src, v);
      static_for<4>([&](auto R) __attribute__((always_inline)) { acc[R] += v[R]; });
    }
    if constexpr (BIAS) {
      float b[4];
      load4(bias + n, b);
      static_for<4>([&](auto R) __attribute__((always_inline)) { acc[R] += b[R]; });
    }
    if constexpr (RES) {
      float r[4];
      load4(residual + m * hidden + n, r);
      static_for<4>([&](auto R) __attribute__((always_inline)) { acc[R] += r[R]; });
    }
    store4(out + m * hidden + n, acc);
  }
}

template <typename IN, typename OUT>
hipError_t launch_typed(const SpPartials& parts, int t, int64_t row0, int64_t rows, int hidden,
                        const void* bias, const void* residual, void* out, hipStream_t stream) {
  const int64_t total = rows * (hidden / 4);
  const int64_t want = (total + 255) / 256;
  const dim3 grid(static_cast<unsigned>(want < 8192 ? want : 8192));
  const IN* b = static_cast<const IN*>(bias);
  const IN* r = static_cast<const IN*>(residual);
  OUT* o = static_cast<OUT*>(out);
  if (b != nullptr && r != nullptr)
    hipLaunchKernelGGL((sp_reduce_kernel<IN, OUT, true, true>), grid, dim3(256), 0, stream, parts, t,
                       row0, rows, hidden, b, r, o);
  else if (b != nullptr)
    hipLaunchKernelGGL((sp_reduce_kernel<IN, OUT, true, false>), grid, dim3(256), 0, stream, parts, t,
                       row0, rows, hidden, b, r, o);
  else if (r != nullptr)
    hipLaunchKernelGGL((sp_reduce_kernel<IN, OUT, false, true>), grid, dim3(256), 0, stream, parts, t,
                       row0, rows, hidden, b, r, o);
  else
    hipLaunchKernelGGL((sp_reduce_kernel<IN, OUT, false, false>), grid, dim3(256), 0, stream, parts,
                       t, row0, rows, hidden, b, r, o);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sp_reduce(const SpPartials& parts, int t, int64_t row0, int64_t rows,
                            int64_t hidden, const void* bias, const void* residual, int in_dt,
                            void* out, int out_dt, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int h = static_cast<int>(hidden);
  if (in_dt == 1)
    return out_dt == 1
               ? launch_typed<uint16_t, uint16_t>(parts, t, row0, rows, h, bias, residual, out, stream)
               : launch_typed<uint16_t, float>(parts, t, row0, rows, h, bias, residual, out, stream);
  return out_dt == 1
             ? launch_typed<float, uint16_t>(parts, t, row0, rows, h, bias, residual, out, stream)
             : launch_typed<float, float>(parts, t, row0, rows, h, bias, residual, out, stream);
}

}  // namespace tpk
